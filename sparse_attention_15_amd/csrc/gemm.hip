// Projections on either side of the DSA path as bf16 MFMA GEMMs on gfx950.
//
//   C[m][n] = sum_k A[m][k] * B[n][k]      (both operands k-contiguous)
//
// batched with strides, bf16 inputs, fp32 accumulation, bf16 or fp32 output.
// The three projections (HF model doc "DeepSeek-V3.2": the indexer's wq_b on
// the query latent, its weights_proj kept out of FP8; sizes from the released
// configuration excerpt on the atlas "DeepSeek-V3.2-Exp" token-ids page):
//   index query:   A = query latent [T][q_lora_rank], B = wq_b [H*D][q_lora_rank]
//   head weights:  A = hidden state [T][dim],         B = weights_proj [H][dim]
//   un-absorption: per head a, A = O[:, a, :] [T][kv_lora_rank] (row stride
//                  NH * kv_lora_rank), B = W_UV[a] [v_head_dim][kv_lora_rank]
//
// Tile kernel (more than 32 rows): 4 waves as 2 x 2, each a TM x TN block of
// 32x32x16 MFMAs; 64-k stages (128 bytes per row) in LDS with chunk c of row r
// stored at c ^ ((r >> 1) & 7), so the rows of an operand read spread over the
// banks; the next stage is loaded into registers while the current one is
// multiplied, one barrier per stage.
// Skinny kernel (at most 32 rows, the decode shapes, which stream the
// weights): one 32 x 32 output tile per work-group; its 4, 8 or 16 waves take
// interleaved 64-k stages through private LDS buffers (no barriers in the
// loop) and add their accumulators through LDS at the end, so that many
// weight loads are in flight per output tile.  When there are too few
// output tiles to fill the chip (the head-weight projection: 64 outputs per
// token over 7168 inputs) and the caller gives a workspace, the k range is
// also split over work-groups, and a second kernel adds the fp32 partials in
// split order.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kGK = 64;                          // k per stage: 8 chunks of 16 bytes per row

// Stage rows are 128 bytes (8 chunks of 16); chunk c of row r is stored at
// c ^ ((r >> 1) & 7).  A 16-lane group of a 16-byte operand read covers 16
// consecutive rows, two per 256-byte bank window: rows of one parity then
// take 8 distinct slots, so the group reads without bank conflicts.
__device__ __forceinline__ int swz8(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ uint32_t tile_off(int r, int c) { return (uint32_t)(r * 128 + ((c ^ swz8(r)) << 4)); }

__device__ __forceinline__ void store_c(const GemmLaunch& g, void* cb, int m, int n, float v) {
  if (g.c_f32)
    static_cast<float*>(cb)[(int64_t)m * g.ldc + n] = v;
  else
    static_cast<uint16_t*>(cb)[(int64_t)m * g.ldc + n] = f32_to_bf16_bits(v);
}

template <int TM, int TN>
__global__ __launch_bounds__(256) void gemm_tile_kernel(GemmLaunch g) {
  constexpr int BM = 2 * TM, BN = 2 * TN, IM = TM / 32, IN = TN / 32;
  constexpr int APT = BM * 8 / 256, BPT = BN * 8 / 256;   // 16-byte chunks per thread and stage
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][(BM + BN) * 128];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
  const uint16_t* A = g.A + (int64_t)blockIdx.z * g.sa;
  const uint16_t* B = g.B + (int64_t)blockIdx.z * g.sb;
  const int nk = (g.K + kGK - 1) / kGK;

  u32x4 ra[APT], rb[BPT];
  auto load = [&](int kt) {
    const int k0 = kt * kGK;
#pragma unroll
    for (int p = 0; p < APT; ++p) {
      const int f = p * 256 + tid, r = f >> 3, k = k0 + 8 * (f & 7);
      const int row = min(m0 + r, g.M - 1);
      ra[p] = k < g.K ? ld16(A + (int64_t)row * g.lda + k) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int p = 0; p < BPT; ++p) {
      const int f = p * 256 + tid, r = f >> 3, k = k0 + 8 * (f & 7);
      const int row = min(n0 + r, g.N - 1);
      rb[p] = k < g.K ? ld16(B + (int64_t)row * g.ldb + k) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int p = 0; p < APT; ++p) {
      const int f = p * 256 + tid;
      st16(&lds[buf][tile_off(f >> 3, f & 7)], ra[p]);
    }
#pragma unroll
    for (int p = 0; p < BPT; ++p) {
      const int f = p * 256 + tid;
      st16(&lds[buf][BM * 128 + tile_off(f >> 3, f & 7)], rb[p]);
    }
  };

  f32x16 acc[IM][IN];
#pragma unroll
  for (int i = 0; i < IM; ++i)
#pragma unroll
    for (int j = 0; j < IN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  load(0);
  store(0);
  __syncthreads();
  const int half = lane >> 5, r32 = lane & 31;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load(kt + 1);
    const uint8_t* base = lds[buf];
#pragma unroll
    for (int s = 0; s < kGK / 16; ++s) {
      const int kc = 2 * s + half;               // this lane's 8 k-values: chunk kc
      u32x4 av[IM], bv[IN];
#pragma unroll
      for (int i = 0; i < IM; ++i) av[i] = ld16(base + tile_off(wm * TM + 32 * i + r32, kc));
#pragma unroll
      for (int j = 0; j < IN; ++j) bv[j] = ld16(base + BM * 128 + tile_off(wn * TN + 32 * j + r32, kc));
#pragma unroll
      for (int i = 0; i < IM; ++i)
#pragma unroll
        for (int j = 0; j < IN; ++j) acc[i][j] = mfma32(av[i], bv[j], acc[i][j]);
    }
    if (kt + 1 < nk) store(buf ^ 1);             // buf ^ 1 was last read before the previous barrier
    __syncthreads();
  }

  void* cb = g.c_f32 ? (void*)(static_cast<float*>(g.C) + (int64_t)blockIdx.z * g.sc)
                     : (void*)(static_cast<uint16_t*>(g.C) + (int64_t)blockIdx.z * g.sc);
#pragma unroll
  for (int i = 0; i < IM; ++i)
#pragma unroll
    for (int j = 0; j < IN; ++j) {
      const int n = n0 + wn * TN + 32 * j + r32;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + wm * TM + 32 * i + 8 * (e >> 2) + 4 * half + (e & 3);
        if (m < g.M && n < g.N) store_c(g, cb, m, n, acc[i][j][e]);
      }
    }
}

template <int NW>   // waves per work-group, each taking every NW-th stage
__global__ __launch_bounds__(NW * 64) void gemm_skinny_kernel(GemmLaunch g) {
  // per wave: one stage of A (32 rows) and B (32 rows), 128 bytes per row
  __shared__ __attribute__((aligned(16))) uint8_t lds[NW][64 * 128];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = blockIdx.x * 32;
  const int bz = blockIdx.z / g.ksplit, kz = blockIdx.z - bz * g.ksplit;
  const uint16_t* A = g.A + (int64_t)bz * g.sa;
  const uint16_t* B = g.B + (int64_t)bz * g.sb;
  const int nk_all = (g.K + kGK - 1) / kGK;
  const int per = (nk_all + g.ksplit - 1) / g.ksplit;   // stages of this split: [k_first, nk)
  const int k_first = kz * per;
  const int nk = min(nk_all, k_first + per);
  uint8_t* mine = lds[wave];

  u32x4 ra[4], rb[4];
  auto load = [&](int kt) {
    const int k0 = kt * kGK;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int f = p * 64 + lane, r = f >> 3, k = k0 + 8 * (f & 7);
      const bool in = k < g.K;
      ra[p] = in ? ld16(A + (int64_t)min(r, g.M - 1) * g.lda + k) : u32x4{0u, 0u, 0u, 0u};
      rb[p] = in ? ld16(B + (int64_t)min(n0 + r, g.N - 1) * g.ldb + k) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  f32x16 acc;
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;
  const int half = lane >> 5, r32 = lane & 31;
  int kt = k_first + wave;
  if (kt < nk) load(kt);
  for (; kt < nk; kt += NW) {
    // the previous stage's operand reads were issued before these writes, and
    // one wave's LDS operations complete in order
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int f = p * 64 + lane;
      st16(mine + tile_off(f >> 3, f & 7), ra[p]);
      st16(mine + 32 * 128 + tile_off(f >> 3, f & 7), rb[p]);
    }
    if (kt + NW < nk) load(kt + NW);
#pragma unroll
    for (int s = 0; s < kGK / 16; ++s) {
      const int kc = 2 * s + half;
      const u32x4 av = ld16(mine + tile_off(r32, kc));
      const u32x4 bv = ld16(mine + 32 * 128 + tile_off(r32, kc));
      acc = mfma32(av, bv, acc);
    }
  }
  // sum the waves' partial tiles through LDS; wave w then finishes the
  // accumulator entries e = w, w + NW, ...
  __syncthreads();                                // every wave is done with its stage buffer
  float* red = reinterpret_cast<float*>(&lds[0][0]);   // [NW][16][64]
#pragma unroll
  for (int e = 0; e < 16; ++e) red[(wave * 16 + e) * 64 + lane] = acc[e];
  __syncthreads();
  void* cb = g.c_f32 ? (void*)(static_cast<float*>(g.C) + (int64_t)bz * g.sc)
                     : (void*)(static_cast<uint16_t*>(g.C) + (int64_t)bz * g.sc);
  float* pp = g.part + ((int64_t)kz * g.batch + bz) * g.M * g.N;   // used when ksplit > 1
  const int n = n0 + r32;
  for (int e = wave; e < 16; e += NW) {
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) v += red[(w * 16 + e) * 64 + lane];
    const int m = 8 * (e >> 2) + 4 * half + (e & 3);
    if (m < g.M && n < g.N) {
      if (g.ksplit > 1) pp[(int64_t)m * g.N + n] = v;
      else store_c(g, cb, m, n, v);
    }
  }
}

// Split-K partials summed in split order (so the result does not depend on
// scheduling), one thread per output.  The partials are loaded 16 at a time
// before any is added: a loop of adds that each wait for their own load ran
// at one memory round trip per split.
__global__ __launch_bounds__(256) void gemm_split_reduce_kernel(GemmLaunch g) {
  constexpr int kLd = 16;
  const int64_t per_b = (int64_t)g.M * g.N;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= per_b * g.batch) return;
  const int bz = (int)(idx / per_b);
  const int64_t mn = idx - bz * per_b;
  const int m = (int)(mn / g.N), n = (int)(mn - (int64_t)m * g.N);
  const float* src = g.part + (int64_t)bz * per_b + mn;
  const int64_t split_stride = (int64_t)g.batch * per_b;
  float v = 0.f;
  for (int k0 = 0; k0 < g.ksplit; k0 += kLd) {
    float t[kLd];
#pragma unroll
    for (int j = 0; j < kLd; ++j) t[j] = k0 + j < g.ksplit ? src[(k0 + j) * split_stride] : 0.f;
#pragma unroll
    for (int j = 0; j < kLd; ++j)
      if (k0 + j < g.ksplit) v += t[j];
  }
  void* cb = g.c_f32 ? (void*)(static_cast<float*>(g.C) + (int64_t)bz * g.sc)
                     : (void*)(static_cast<uint16_t*>(g.C) + (int64_t)bz * g.sc);
  store_c(g, cb, m, n, v);
}

// Big-tile kernel (many rows, k a multiple of 64): a 256 x BN output tile,
// 4 waves as 2 x 2 of 128 x BN/2 (4 x BN/64 tiles of 32x32x16 MFMAs).  At
// 128 x 128 tiles the L2 -> CU traffic per flop matches the chip's balance
// point; 256 x BN halves it.  64-k stages move global -> LDS by LDS-DMA (no
// registers), with the chunk permutation applied on the source side; NST stages in a ring, NST - 1 in flight, one barrier per stage.  The
// output leaves through LDS, 16 bytes per lane along rows.
template <int BN, int NST, int W>
__global__ __launch_bounds__(W * 64, W / 4) void gemm_big_kernel(GemmLaunch g) {
  constexpr int BM = 256, TM = 128, TN = BN / (W / 2), IM = TM / 32, IN = TN / 32;
  constexpr int STAGE = (BM + BN) * 128;          // bytes per stage: rows of 64 bf16
  constexpr int NCOPY = STAGE / 1024;             // 1 KB copies per stage
  constexpr int CPW = NCOPY / W;                  // per wave
  constexpr int ACOPY = BM * 128 / 1024;          // the first ACOPY copies fill A rows
  static_assert(NCOPY % W == 0, "copies split evenly over the waves");
  __shared__ __attribute__((aligned(16))) uint8_t lds[NST * STAGE];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / (W / 2), wn = wave % (W / 2);
  // Batch index fastest in launch order: consecutive work-groups take the
  // same tile of consecutive batch entries, which for the per-head
  // un-absorption are neighbouring 1 KB pieces of the same token rows (one
  // stream instead of 128 strided ones).  Batch 1 keeps the grid order.
  const int lin = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
  const int bz = lin % g.batch, rest = lin / g.batch;
  const int bx = rest % gridDim.x, by = rest / gridDim.x;
  const int n0 = bx * BN, m0 = by * BM;
  const int nk = g.K / kGK;
  // uniform bases at this tile's first rows (per-lane offsets stay small)
  const uint8_t* abase = reinterpret_cast<const uint8_t*>(g.A + (int64_t)bz * g.sa + (int64_t)m0 * g.lda);
  const uint8_t* bbase = reinterpret_cast<const uint8_t*>(g.B + (int64_t)bz * g.sb + (int64_t)n0 * g.ldb);
  // copy c = wave * CPW + k (uniform) fills A rows if c < ACOPY, else B rows
  uint32_t off[CPW];
#pragma unroll
  for (int k = 0; k < CPW; ++k) {
    const int f = 64 * (wave * CPW + k) + lane;   // LDS slot of the stage
    const int r = f >> 3, c = (f & 7) ^ swz8(r);  // row, global chunk stored there
    if (wave * CPW + k < ACOPY) off[k] = (uint32_t)((min(m0 + r, g.M - 1) - m0) * g.lda * 2 + 16 * c);
    else off[k] = (uint32_t)((min(n0 + r - BM, g.N - 1) - n0) * g.ldb * 2 + 16 * c);
  }
  const uint32_t lds0 = lds_addr(lds);
  auto issue = [&](int st) {
    const uint32_t dst = __builtin_amdgcn_readfirstlane(lds0 + (st % NST) * STAGE + 1024 * wave * CPW);
#pragma unroll
    for (int k = 0; k < CPW; ++k) {
      const uint8_t* gb = (wave * CPW + k < ACOPY ? abase : bbase) + (int64_t)st * (kGK * 2);
      lds_dma16<false>(gb, off[k], dst + 1024 * k);
    }
  };

  f32x16 acc[IM][IN];
#pragma unroll
  for (int i = 0; i < IM; ++i)
#pragma unroll
    for (int j = 0; j < IN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int half = lane >> 5, r32 = lane & 31;
#pragma unroll
  for (int j = 0; j < NST - 1; ++j)
    if (j < nk) issue(j);
  for (int st = 0; st < nk; ++st) {
    // this wave's copies of stage st landed once at most the later issued
    // stages' copies are outstanding
    const int ahead = min(nk - 1 - st, NST - 2);
    if (ahead >= 2) wait_vmcnt<2 * CPW>();
    else if (ahead == 1) wait_vmcnt<CPW>();
    else wait_vmcnt<0>();
    __syncthreads();                              // everyone's; stage st-1 is no longer read
    if (st + NST - 1 < nk) issue(st + NST - 1);  // into the buffer of stage st-1
    const uint8_t* base = lds + (st % NST) * STAGE;
#pragma unroll
    for (int s = 0; s < kGK / 16; ++s) {
      const int kc = 2 * s + half;
      u32x4 av[IM], bv[IN];
#pragma unroll
      for (int i = 0; i < IM; ++i) av[i] = ld16(base + tile_off(wm * TM + 32 * i + r32, kc));
#pragma unroll
      for (int j = 0; j < IN; ++j) bv[j] = ld16(base + BM * 128 + tile_off(wn * TN + 32 * j + r32, kc));
#pragma unroll
      for (int i = 0; i < IM; ++i)
#pragma unroll
        for (int j = 0; j < IN; ++j) acc[i][j] = mfma32(av[i], bv[j], acc[i][j]);
    }
  }

  // epilogue: per 32-row slice of the wave tile, rows of TN values through a
  // private LDS area, then 16-byte stores along the rows
  __syncthreads();                                // the stages are free
  const int esz = g.c_f32 ? 4 : 2;
  const int pitch = TN * 4 + 16;                  // bytes per staged row (fp32 room, padded)
  uint8_t* ebuf = lds + wave * 32 * pitch;
  uint8_t* cb = static_cast<uint8_t*>(g.C) + ((int64_t)bz * g.sc) * esz;
  const int row_bytes = TN * esz, chunks = 32 * row_bytes / 16;
#pragma unroll
  for (int i = 0; i < IM; ++i) {
#pragma unroll
    for (int j = 0; j < IN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int rr = 8 * (e >> 2) + 4 * half + (e & 3), cc = 32 * j + r32;
        if (g.c_f32) *reinterpret_cast<float*>(ebuf + rr * pitch + cc * 4) = acc[i][j][e];
        else *reinterpret_cast<uint16_t*>(ebuf + rr * pitch + cc * 2) = f32_to_bf16_bits(acc[i][j][e]);
      }
    __builtin_amdgcn_s_waitcnt(0xc07f);           // lgkmcnt(0): this wave's LDS writes are done
    for (int q = lane; q < chunks; q += 64) {
      const int rr = q / (row_bytes / 16), cq = q - rr * (row_bytes / 16);
      const int m = m0 + wm * TM + 32 * i + rr;
      const int n = n0 + wn * TN + cq * (16 / esz);
      if (m < g.M && n < g.N) st16(cb + ((int64_t)m * g.ldc + n) * esz, ld16(ebuf + rr * pitch + cq * 16));
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);           // reads done before the next slice overwrites
  }
}

}  // namespace

int gemm_ksplit(int M, int N, int K, int batch, size_t* bytes) {
  *bytes = 0;
  if (M > 32) return 1;
  const int64_t wgs = (int64_t)((N + 31) / 32) * batch;
  const int nk = (K + kGK - 1) / kGK;
  if (wgs >= 64 || nk < 16) return 1;
  // about 128 work-groups, each with at least 4 stages (one per wave)
  int ks = (int)(128 / wgs);
  ks = min(ks, nk / 4);
  if (ks < 2) return 1;
  *bytes = (size_t)ks * batch * M * N * sizeof(float);
  return ks;
}

hipError_t launch_gemm_bt(const GemmLaunch& g, hipStream_t s) {
  if (g.ksplit > 1) {                            // skinny shapes only (see gemm_ksplit)
    dim3 grid((g.N + 31) / 32, 1, g.batch * g.ksplit);
    hipLaunchKernelGGL(gemm_skinny_kernel<4>, grid, dim3(256), 0, s, g);
    const int64_t outs = (int64_t)g.M * g.N * g.batch;
    hipLaunchKernelGGL(gemm_split_reduce_kernel, dim3((unsigned)((outs + 255) / 256)), dim3(256), 0, s, g);
    return hipGetLastError();
  }
  if (g.M <= 32) {
    // few output tiles: more waves per tile, so that enough weight loads are
    // in flight per CU
    dim3 grid((g.N + 31) / 32, 1, g.batch);
    const int64_t wgs = (int64_t)grid.x * g.batch;
    if (wgs >= 1024)
      hipLaunchKernelGGL(gemm_skinny_kernel<4>, grid, dim3(256), 0, s, g);
    else if (wgs >= 64)
      hipLaunchKernelGGL(gemm_skinny_kernel<8>, grid, dim3(512), 0, s, g);
    else
      hipLaunchKernelGGL(gemm_skinny_kernel<16>, grid, dim3(1024), 0, s, g);
  } else if (g.M >= 256 && g.N >= 128 && g.K % kGK == 0 && g.N % 8 == 0 && g.ldc % 8 == 0 &&
             (g.sc * (g.c_f32 ? 4 : 2)) % 16 == 0 && (reinterpret_cast<uintptr_t>(g.C) & 15) == 0) {
    if (g.batch == 1 && g.N >= 1024) {
      dim3 grid((g.N + 255) / 256, (g.M + 255) / 256, g.batch);
      hipLaunchKernelGGL((gemm_big_kernel<256, 2, 8>), grid, dim3(512), 0, s, g);
    } else {
      dim3 grid((g.N + 127) / 128, (g.M + 255) / 256, g.batch);
      hipLaunchKernelGGL((gemm_big_kernel<128, 3, 8>), grid, dim3(512), 0, s, g);
    }
  } else if (g.M >= 128 && g.N >= 128) {
    dim3 grid((g.N + 127) / 128, (g.M + 127) / 128, g.batch);
    hipLaunchKernelGGL((gemm_tile_kernel<64, 64>), grid, dim3(256), 0, s, g);
  } else {
    dim3 grid((g.N + 63) / 64, (g.M + 63) / 64, g.batch);
    hipLaunchKernelGGL((gemm_tile_kernel<32, 32>), grid, dim3(256), 0, s, g);
  }
  return hipGetLastError();
}

}  // namespace dsa
