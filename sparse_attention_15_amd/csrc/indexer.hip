// Lightning-indexer scores on gfx950.
//
// For query (b, i) at position p and key s <= p:
//     I[s] = sum_h w[h] * max(0, q_h . k_s)
// (HF model doc "DeepSeek-V3.2", section "DeepSeek Sparse Attention (DSA)",
// item 1: a scorer with few heads rates every earlier key; the index keys are
// one head of index_head_dim per token; per-query head weights come from the
// indexer's weights_proj.  The ReLU-gated, weighted head sum is the reading
// this library implements.)
//
// bf16 / fp8 kernels (H = 64, D = 128): the per-head dot products are an MFMA
// GEMM with heads on the M axis (4 tiles of 16) and keys on the N axis, so
// the ReLU-weighted head reduction happens in registers: 16 values per lane,
// then two cross-lane adds.  Keys are read once per query group: through a
// per-wave LDS-DMA ring of whole key rows for decode-shaped launches, through
// an LDS-DMA ring of swizzled 64-key tiles shared by 8 queries for
// prefill-shaped ones (4 slots for bf16, 6 for FP8).
// FP8 (E4M3 codes + ue8m0 row scales): the MFMA consumes raw codes; the
// query-row scales fold into the head weights and the key scale multiplies
// the head sum.  Both are powers of two and ReLU is positively homogeneous,
// so this equals scoring the dequantised values.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr float kNegInf = -__builtin_inff();

// ------------------------------------------------------------- fp32 -------
// One thread per key; the query's H x D block and head weights sit in LDS.
__global__ __launch_bounds__(256) void idx_f32_kernel(IndexLaunch a) {
  extern __shared__ float sm[];
  const int H = a.H, D = a.D;
  float* qs = sm;
  float* ws = sm + H * D;
  const int row = blockIdx.y;
  const int b = row / a.q_count;
  const int i = a.q_begin + row % a.q_count;
  const int n = a.Lk - a.Lq + i + 1;
  const int s0 = blockIdx.x * 256;
  if (s0 >= n && !a.write_masked) return;
  const int64_t qrow = (int64_t)b * a.Lq + i;
  const float* qg = static_cast<const float*>(a.q) + qrow * H * D;
  for (int e = threadIdx.x; e < H * D; e += 256) qs[e] = qg[e];
  for (int e = threadIdx.x; e < H; e += 256) ws[e] = a.w[qrow * H + e];
  __syncthreads();
  const int s = s0 + threadIdx.x;
  if (s >= a.Lk) return;
  float* out = a.scores + (int64_t)row * a.row_stride;
  if (s >= n) {
    if (a.write_masked) out[s] = kNegInf;
    return;
  }
  const float* kr = static_cast<const float*>(a.k) + ((int64_t)b * a.Lc + s) * D;
  float acc = 0.f;
  for (int h = 0; h < H; ++h) {
    float x = 0.f;
    for (int d = 0; d < D; ++d) x = fmaf(qs[h * D + d], kr[d], x);
    acc = fmaf(ws[h], fmaxf(x, 0.f), acc);
  }
  out[s] = acc;
}

// -------------------------------------------------- MFMA building blocks ---
// Lane l of a wave works on column r = l % 16 of a 16-wide key tile and on
// k-group g = l / 16.  bf16: k-step t (0..3) covers dims 32t + 8g .. +8.
// fp8: one 16x16x128 MFMA covers all 128 dims; group g holds dims 32g .. +32.
constexpr int kH = 64;
constexpr int kD = 128;

template <bool FP8> struct QFrag;
template <> struct QFrag<false> { u32x4 v[4][4]; };  // [m-tile][k-step]
template <> struct QFrag<true>  { i32x8 v[4]; };     // [m-tile]
template <bool FP8> struct KFrag;
template <> struct KFrag<false> { u32x4 v[4]; };     // [k-step]
template <> struct KFrag<true>  { i32x8 v; };

__device__ __forceinline__ i32x8 join(u32x4 lo, u32x4 hi) {
  i32x8 r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  return r;
}

// Query fragments and the 16 head weights this lane needs (heads 16m + 4g + j).
template <bool FP8>
__device__ __forceinline__ void load_query(const IndexLaunch& a, int64_t qrow, int lane,
                                           QFrag<FP8>& q, float (&wv)[16]) {
  const int r = lane & 15, g = lane >> 4;
  if constexpr (!FP8) {
    const uint8_t* base = static_cast<const uint8_t*>(a.q) + qrow * (kH * kD * 2);
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int t = 0; t < 4; ++t)
        q.v[m][t] = ld16(base + ((16 * m + r) * kD + 32 * t + 8 * g) * 2);
  } else {
    const uint8_t* base = static_cast<const uint8_t*>(a.q) + qrow * (kH * kD);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint8_t* p = base + (16 * m + r) * kD + 32 * g;
      q.v[m] = join(ld16(p), ld16(p + 16));
    }
  }
  const float* w = a.w + qrow * kH;
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int h = 16 * m + 4 * g + j;
      float wh = w[h];
      if constexpr (FP8) wh *= ue8m0_to_f32(a.q_scale[qrow * kH + h]);
      wv[4 * m + j] = wh;
    }
}

// max(x, 0).  FP8 tiles take half the MFMA time of bf16 ones, so their
// ReLU-weighted head sum sets the pace: there it is one median-of-three
// (0, x, FLT_MAX) instead of fmaxf, which first quiets a possible
// signalling NaN in the MFMA result with a second max (the bound only
// differs at +inf, which a sum of finite fp8 products in fp32 does not
// reach).  bf16 keeps fmaxf: measured faster there (its schedule).
template <bool FP8>
__device__ __forceinline__ float relu(float x) {
  if constexpr (FP8) return __builtin_amdgcn_fmed3f(x, 0.f, 3.402823466e38f);
  else return fmaxf(x, 0.f);
}

// This lane's part of the scores of one 16-key tile for one query: the
// ReLU-weighted sum over its 16 heads (16m + 4g + j) for key r; the four
// k-groups' parts add up to the score.
template <bool FP8>
__device__ __forceinline__ float tile_partial(const QFrag<FP8>& q, const KFrag<FP8>& kf, const float (&wv)[16]) {
  f32x4 acc[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
  if constexpr (!FP8) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int m = 0; m < 4; ++m) acc[m] = mfma16(q.v[m][t], kf.v[t], acc[m]);
  } else {
    // Scale operands 0 select the unscaled encoding (v_mfma_f32_16x16x128_f8f6f4),
    // which issues faster than the scaled one; both give the plain E4M3
    // products (bit-identical on gfx950).
#pragma unroll
    for (int m = 0; m < 4; ++m)
      acc[m] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(q.v[m], kf.v, acc[m], 0, 0, 0, 0, 0, 0);
  }
  // Two independent accumulation chains (head tiles 0-1 and 2-3), so that
  // the dependent FMAs of one can issue between those of the other.
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      s0 = fmaf(wv[4 * m + j], relu<FP8>(acc[m][j]), s0);
      s1 = fmaf(wv[4 * m + 8 + j], relu<FP8>(acc[m + 2][j]), s1);
    }
  return s0 + s1;
}

// Scores of one 16-key tile for one query: returns the score of key r in
// every lane (all four k-groups hold the same value after the reduction).
template <bool FP8>
__device__ __forceinline__ float tile_score(const QFrag<FP8>& q, const KFrag<FP8>& kf, const float (&wv)[16]) {
  float s = tile_partial<FP8>(q, kf, wv);
  // sum over the four 16-lane groups: rows l and l ^ 16 through
  // v_permlane16_swap, then the two halves of the wave through
  // v_permlane32_swap (no LDS round trips)
  float r0, r1;
  xor16_pair(s, r0, r1);
  s = r0 + r1;
  float lo, hi;
  xor32_pair(s, lo, hi);
  return lo + hi;
}

// Four tiles' parts p[t] (lane group g holds group g's part of each) ->
// lane group g returns the score of tile g: a reduce-scatter in two swaps.
// v_permlane16_swap(a, b) leaves, in even rows, (own a, partner's a) and, in
// odd rows, (partner's b, own b); v_permlane32_swap does the same for the
// wave halves.  Sums come out as (g0 + g1) + (g2 + g3), as in tile_score.
__device__ __forceinline__ float reduce4(float p0, float p1, float p2, float p3) {
  uint32_t a0 = __builtin_bit_cast(uint32_t, p0), a1 = __builtin_bit_cast(uint32_t, p1);
  uint32_t b0 = __builtin_bit_cast(uint32_t, p2), b1 = __builtin_bit_cast(uint32_t, p3);
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\tv_permlane16_swap_b32 %2, %3"
               : "+v"(a0), "+v"(a1), "+v"(b0), "+v"(b1));
  // pair sums over rows (0, 1) and (2, 3): even rows hold tiles 0 (a) and
  // 2 (b), odd rows tiles 1 and 3
  uint32_t ta = __builtin_bit_cast(uint32_t, __builtin_bit_cast(float, a0) + __builtin_bit_cast(float, a1));
  uint32_t tb = __builtin_bit_cast(uint32_t, __builtin_bit_cast(float, b0) + __builtin_bit_cast(float, b1));
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(ta), "+v"(tb));
  return __builtin_bit_cast(float, ta) + __builtin_bit_cast(float, tb);
}

// ------------------------------------------- decode: candidate lists -------
// The chunk's candidate list for the filtered top-k (256 threads; the
// chunk's nk scores in sc; hist: 4096 + 8 words of free LDS).  Every
// visible key of the chunk whose 12-bit key prefix (sign, exponent, three
// mantissa bits) lies above the cutoff bin goes to the list, in position
// order; the cutoff is the highest bin at which more than cand_m keys would
// be listed (-1 when the chunk has at most cand_m keys).  The top-k then
// only needs the lists: if the K-th largest listed key lies in a bin above
// every chunk's cutoff, every key at least as large as it is listed, so the
// lists hold the whole selection.
__device__ void chunk_candidates(const IndexLaunch& a, int row, int nk, const float* sc, uint32_t* hist) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t* red = hist + 4096;
  const int M = a.cand_m;
  const int64_t lst = (int64_t)row * gridDim.x + blockIdx.x;
  // positions 8 tid .. 8 tid + 7 of the chunk
  uint32_t k[8];
  {
    const f32x4 v0 = *reinterpret_cast<const f32x4*>(sc + 8 * tid);
    const f32x4 v1 = *reinterpret_cast<const f32x4*>(sc + 8 * tid + 4);
    const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) k[e] = 8 * tid + e < nk ? order_key(v[e]) : 0u;
  }
  int cut = -1;
  if (nk > M) {                                  // uniform
#pragma unroll
    for (int q = 0; q < 4; ++q) st16(hist + 4 * (tid + 256 * q), u32x4{0u, 0u, 0u, 0u});
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (k[e]) atomicAdd(&hist[k[e] >> 20], 1u);
    __syncthreads();
    // thread t holds bins 4095 - 16t - j, j = 0..15 (from the top down)
    const int top = 4095 - 16 * tid;
    uint32_t c[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x4 h = *reinterpret_cast<const u32x4*>(hist + top - 4 * q - 3);
      c[4 * q] = h.w;
      c[4 * q + 1] = h.z;
      c[4 * q + 2] = h.y;
      c[4 * q + 3] = h.x;
    }
    uint32_t tot = 0u;
#pragma unroll
    for (int j = 0; j < 16; ++j) tot += c[j];
    const uint32_t incl = wave_incl_scan(tot);
    if (lane == 63) red[4 + wave] = incl;
    __syncthreads();
    uint32_t run = incl - tot;                   // keys in the bins above mine
    for (int w = 0; w < wave; ++w) run += red[4 + w];
    if (run <= (uint32_t)M && run + tot > (uint32_t)M) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if (run + c[j] > (uint32_t)M) {
          red[0] = (uint32_t)(top - j);
          break;
        }
        run += c[j];
      }
    }
    __syncthreads();
    cut = (int)red[0];
  }
  uint32_t take = 0u;
#pragma unroll
  for (int e = 0; e < 8; ++e) take |= (k[e] != 0u && (int)(k[e] >> 20) > cut) ? (1u << e) : 0u;
  const uint32_t cnt = __builtin_popcount(take);
  const uint32_t incl = wave_incl_scan(cnt);
  if (lane == 63) red[4 + wave] = incl;
  __syncthreads();
  uint32_t off = incl - cnt, total = 0u;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    off += w < wave ? red[4 + w] : 0u;
    total += red[4 + w];
  }
  uint32_t* keys = a.cand_keys + lst * kCandCap;
  uint16_t* offs = a.cand_offs + lst * kCandCap;
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (take & (1u << e)) {
      keys[off] = k[e];
      offs[off] = (uint16_t)(8 * tid + e);
      ++off;
    }
  if (tid == 0) *reinterpret_cast<int2*>(a.cand_hdr + 2 * lst) = int2{(int)total, cut};
}

// ------------------------------------------------------ decode shape -------
// grid (ceil(Lk / 2048), B * q_count), 4 waves; the work-group walks the
// 16-key tiles of keys [c0, c0 + 2048) of its query in order, tile t going
// to wave t % 4, so the four waves read one contiguous stream.  Each wave's
// tiles pass through a private 3-stage LDS ring filled by LDS-DMA
// (global_load_lds): each copy instruction moves whole 256-byte (bf16) or
// 128-byte (fp8) key rows, so every request is a full cache line, and no
// registers hold data in flight.  Within a staged row the 16-byte chunks are
// XOR-permuted by the row index, which makes the MFMA operand reads
// conflict-free.  Scores collect in LDS and leave with coalesced stores
// after one barrier, so the vector-memory counter only tracks the copies.
constexpr int kDecChunk = 2048;                  // keys per work-group
// Three stages (two in flight while one is consumed) at two work-groups per
// CU: 32 x 32K decode indexer 46.0 -> 45.4 us against four stages.
constexpr int kDecRing = 3;

template <bool FP8>
__global__ __launch_bounds__(256, 2) void idx_decode_kernel(IndexLaunch a) {
  constexpr int ROWB = FP8 ? kD : 2 * kD;        // bytes per key row
  constexpr int CPR = ROWB / 16;                 // 16-byte chunks per row
  constexpr int TK = 16;                         // keys per stage
  constexpr int STG = TK * ROWB;                 // bytes per stage
  constexpr int NDMA = STG / 1024;               // copy instructions per stage
  __shared__ __attribute__((aligned(16))) uint8_t ring[4][kDecRing][STG];
  __shared__ __attribute__((aligned(16))) float sc[kDecChunk];
  __shared__ __attribute__((aligned(16))) uint8_t kscale[FP8 ? kDecChunk : 16];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = blockIdx.y;
  const int b = row / a.q_count;
  const int i = a.q_begin + row % a.q_count;
  const int n = a.Lk - a.Lq + i + 1;
  const int c0 = blockIdx.x * kDecChunk;
  const int c1 = min(c0 + kDecChunk, a.Lk);
  const int cn = min(c1, n);
  float* out = a.scores + (int64_t)row * a.row_stride;
  if (a.write_masked) {
    for (int s = max(c0, n) + tid; s < c1; s += 256) out[s] = kNegInf;
    wait_vmcnt<0>();
  }
  if (a.zero_hist && blockIdx.x == 0) {          // the sliced top-k's row head
    u32x4* h = reinterpret_cast<u32x4*>(a.zero_hist + (int64_t)row * kTopkRowHeadWords);
    for (int j = tid; j < kTopkRowHeadWords / 4; j += 256) h[j] = u32x4{0u, 0u, 0u, 0u};
    wait_vmcnt<0>();
  }
  if (c0 >= cn) {                                // uniform over the work-group
    if (a.cand_m && tid == 0)                     // no visible key: an empty list
      *reinterpret_cast<int2*>(a.cand_hdr + 2 * ((int64_t)row * gridDim.x + blockIdx.x)) = int2{0, -1};
    return;
  }
  const int nk = cn - c0;
  const int ntile = (nk + TK - 1) / TK;
  const int nst = (ntile - wave + 3) / 4;        // my tiles: wave, wave + 4, ...

  const int64_t qrow = (int64_t)b * a.Lq + i;
  const uint8_t* kbase = static_cast<const uint8_t*>(a.k) + (int64_t)b * a.Lc * ROWB;   // wave-uniform

  // copy k of a stage fills LDS slots 64k + lane: row slot/CPR, stored
  // position slot%CPR, holding global chunk position ^ (row % CPR)
  int drow[NDMA], dchk[NDMA];
#pragma unroll
  for (int k = 0; k < NDMA; ++k) {
    const int slot = 64 * k + lane;
    drow[k] = slot / CPR;
    dchk[k] = (slot % CPR) ^ (drow[k] & (CPR - 1));
  }
  const uint32_t ring_lds = lds_addr(&ring[wave][0][0]);
  auto issue = [&](int st) {
    const int k0 = c0 + (4 * st + wave) * TK;
    const uint32_t dst = __builtin_amdgcn_readfirstlane(ring_lds + (st % kDecRing) * STG);
#pragma unroll
    for (int k = 0; k < NDMA; ++k) {
      const int key = min(k0 + drow[k], a.Lk - 1);   // rows past the end repeat the last key
      lds_dma16(kbase, (uint32_t)key * ROWB + dchk[k] * 16, dst + 1024 * k);
    }
  };
  // first stages in flight before the query loads, so both latencies overlap
#pragma unroll
  for (int st = 0; st < kDecRing - 1; ++st)
    if (st < nst) issue(st);
  if constexpr (FP8) {
    const uint8_t* ks = a.k_scale + (int64_t)b * a.Lc;
    for (int j = tid; j < nk; j += 256) kscale[j] = ks[c0 + j];
  }
  QFrag<FP8> q;
  float wv[16];
  load_query<FP8>(a, qrow, lane, q, wv);
  // Wait for everything issued so far (the query loads are the youngest), so
  // that inside the loop only the copies use the vector-memory counter.
  wait_vmcnt<0>();
  if constexpr (FP8) __syncthreads();            // the key scales are in LDS
  if constexpr (!FP8) {
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int t = 0; t < 4; ++t) asm volatile("" : "+v"(q.v[m][t]));
  } else {
#pragma unroll
    for (int m = 0; m < 4; ++m) asm volatile("" : "+v"(q.v[m]));
  }
#pragma unroll
  for (int e = 0; e < 16; ++e) asm volatile("" : "+v"(wv[e]));

  const int r16 = lane & 15, g = lane >> 4;
  for (int st = 0; st < nst; ++st) {
    // stage st is complete when at most the later in-flight stages remain
    static_assert(kDecRing == 3, "one later stage in flight at the wait");
    if (st + 1 < nst) wait_vmcnt<NDMA>();
    else wait_vmcnt<0>();
    asm volatile("" ::: "memory");
    // the slot of stage st-1 is free again (its reads have returned)
    if (st + kDecRing - 1 < nst) issue(st + kDecRing - 1);
    const uint8_t* lrow = &ring[wave][st % kDecRing][r16 * ROWB];
    KFrag<FP8> kf;
    if constexpr (!FP8) {
#pragma unroll
      for (int t = 0; t < 4; ++t) kf.v[t] = ld16(lrow + (((4 * t + g) ^ r16) * 16));
    } else {
      kf.v = join(ld16(lrow + (((2 * g) ^ (r16 & 7)) * 16)), ld16(lrow + (((2 * g + 1) ^ (r16 & 7)) * 16)));
    }
    float s = tile_score<FP8>(q, kf, wv);
    const int j = (4 * st + wave) * TK + lane;
    if (lane < TK) {
      if constexpr (FP8) s *= ue8m0_to_f32(kscale[min(j, kDecChunk - 1)]);
      sc[j] = s;
    }
  }
  // coalesced stores of the work-group's scores
  __syncthreads();
  for (int j = tid; j < nk; j += 256) out[c0 + j] = sc[j];
  // the key rings are free now (every wave has passed its last stage)
  static_assert(sizeof(ring) >= (4096 + 8) * 4, "the candidate histogram fits in the rings");
  if (a.cand_m) chunk_candidates(a, row, nk, sc, reinterpret_cast<uint32_t*>(&ring[0][0][0]));
}

// ----------------------------------------------------- prefill shape -------
// grid (ceil(q_count / QB), ksplit, B), QB waves = QB consecutive queries.
// The block walks 64-key tiles kt = blockIdx.y, +ksplit, ... up to the last
// query's causal limit.  Tiles stream through an LDS ring filled by LDS-DMA
// (whole key rows per copy instruction, chunks XOR-permuted by row so the
// MFMA operand reads are conflict-free); each tile is consumed by all QB
// waves.  bf16: a 4-deep ring and one barrier per tile; FP8 tiles take half
// the time, so they go two per barrier through a 6-deep ring.  Either way two
// tiles are in flight while the current ones are consumed.

template <bool FP8, int QB>
__global__ __launch_bounds__(QB * 64) void idx_prefill_kernel(IndexLaunch a, int ksplit) {
  constexpr int TK = 64;
  constexpr int ROWB = FP8 ? kD : 2 * kD;        // bytes per key row
  constexpr int CPR = ROWB / 16;                  // 16-byte chunks per row
  constexpr int STG = TK * ROWB;                  // bytes per tile
  constexpr int NDMA = STG / 1024;                // copy instructions per tile
  static_assert(NDMA % QB == 0 || QB % NDMA == 0, "tile copies must split evenly over the waves");
  constexpr int DPW = NDMA >= QB ? NDMA / QB : 1; // copies per wave (waves >= NDMA issue none)
  constexpr int STEP = FP8 ? 2 : 1;               // tiles per barrier
  constexpr int RING = 2 * STEP + 2;              // ring slots
  __shared__ __attribute__((aligned(16))) uint8_t ring[RING][STG];
  // FP8: the tile's 64 key-scale bytes, one dword per key, copied by wave
  // QB - 1 next to its share of the tile (no register load whose wait would
  // also wait for the tiles in flight)
  __shared__ __attribute__((aligned(16))) uint32_t kscl[FP8 ? RING : 1][TK];

  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int qb = gridDim.x - 1 - blockIdx.x;      // longest rows first
  const int b = blockIdx.z;
  const int ii = qb * QB + wave;
  const bool active = ii < a.q_count;
  const int i = a.q_begin + ii;
  const int p = a.Lk - a.Lq + i;
  const int last = min(qb * QB + QB, a.q_count) - 1;
  const int n_max = a.Lk - a.Lq + a.q_begin + last + 1;
  const int ntiles = (n_max + TK - 1) / TK;
  const int row = b * a.q_count + ii;
  float* out = a.scores + (int64_t)row * a.row_stride;
  const uint8_t* kbase = static_cast<const uint8_t*>(a.k) + (int64_t)b * a.Lc * ROWB;   // uniform
  const uint8_t* ks = FP8 ? a.k_scale + (int64_t)b * a.Lc : nullptr;

  // this block's tiles: kt = blockIdx.y + ksplit * j, j < nj
  const int nj = blockIdx.y < ntiles ? (ntiles - 1 - blockIdx.y) / ksplit + 1 : 0;
  // copy c (wave's k-th, c = wave * DPW + k) fills LDS slots 64c + lane: row
  // slot/CPR, stored position slot%CPR, holding global chunk position ^ row
  int drow[DPW], dchk[DPW];
#pragma unroll
  for (int k = 0; k < DPW; ++k) {
    const int slot = 64 * (wave * DPW + k) + lane;
    drow[k] = slot / CPR;
    dchk[k] = (slot % CPR) ^ (drow[k] & (CPR - 1));
  }
  const bool copies = wave * DPW < NDMA;
  static_assert(!FP8 || (QB - 1) * DPW < NDMA, "the scale-copying wave also copies key rows");
  const bool scl = FP8 && wave == QB - 1;         // copies DPW + 1 per tile
  const uint32_t ring_lds = lds_addr(&ring[0][0]);
  const uint32_t kscl_lds = lds_addr(&kscl[0][0]);
  auto issue = [&](int j) {
    if (!copies) return;
    const int k0 = (blockIdx.y + ksplit * j) * TK;
    const uint32_t dst = __builtin_amdgcn_readfirstlane(ring_lds + (j % RING) * STG);
#pragma unroll
    for (int k = 0; k < DPW; ++k) {
      const int key = min(k0 + drow[k], a.Lk - 1);   // rows past the end repeat the last key
      lds_dma16(kbase, (uint32_t)key * ROWB + dchk[k] * 16, dst + 1024 * (wave * DPW + k));
    }
    if (scl)
      lds_dma_u8(ks, (uint32_t)min(k0 + lane, a.Lk - 1),
                 __builtin_amdgcn_readfirstlane(kscl_lds + (j % RING) * (TK * 4)));
  };
#pragma unroll
  for (int j = 0; j < RING - STEP; ++j)
    if (j < nj) issue(j);

  QFrag<FP8> q;
  float wv[16];
  if (active) load_query<FP8>(a, (int64_t)b * a.Lq + i, lane, q, wv);
  wait_vmcnt<0>();                                // prologue loads complete; only copies and
                                                  // score stores use the counter from here on

  const int r16 = lane & 15, g = lane >> 4;
  // wait until at most `later` tiles of this wave's copies are in flight
  // (score stores, which may also be outstanding, only make the wait stricter)
  auto wait_tiles = [&](int later) {
    if (scl) {
      if (later >= 2) wait_vmcnt<2 * (DPW + 1)>();
      else if (later == 1) wait_vmcnt<DPW + 1>();
      else wait_vmcnt<0>();
    } else if (copies) {
      if (later >= 2) wait_vmcnt<2 * DPW>();
      else if (later == 1) wait_vmcnt<DPW>();
      else wait_vmcnt<0>();
    }
  };
  auto tile_scores = [&](int j) {                 // this wave's scores of tile j
    const int kt = blockIdx.y + ksplit * j;
    if (!active || kt * TK > p) return;
    const uint8_t* tile = &ring[j % RING][0];
    float part[TK / 16];                           // this lane's parts of the 4 sub-tiles
#pragma unroll
    for (int st = 0; st < TK / 16; ++st) {
      const int rr = 16 * st + r16;
      const uint8_t* lrow = tile + rr * ROWB;
      KFrag<FP8> kf;
      if constexpr (!FP8) {
#pragma unroll
        for (int t = 0; t < 4; ++t) kf.v[t] = ld16(lrow + (((4 * t + g) ^ (rr & 15)) * 16));
      } else {
        kf.v = join(ld16(lrow + (((2 * g) ^ (rr & 7)) * 16)), ld16(lrow + (((2 * g + 1) ^ (rr & 7)) * 16)));
      }
      part[st] = tile_partial<FP8>(q, kf, wv);
    }
    // lane 16 g + r16 gets the score of key 16 g + r16
    float mine = reduce4(part[0], part[1], part[2], part[3]);
    // one 256-byte store per tile and wave
    const int key = kt * TK + lane;
    if (key <= p) {
      if constexpr (FP8) mine *= ue8m0_to_f32(kscl[j % RING][lane]);
      out[key] = mine;
    }
  };
  for (int j0 = 0; j0 < nj; j0 += STEP) {
    // tiles j0 .. j0 + STEP - 1 complete; tiles up to j0 + RING - STEP - 1
    // were issued
    wait_tiles(max(0, min(nj, j0 + RING - STEP) - (j0 + STEP)));
    __builtin_amdgcn_s_barrier();                 // every wave's copies landed; the previous tiles are free
    asm volatile("" ::: "memory");
#pragma unroll
    for (int u = 0; u < STEP; ++u)
      if (j0 + RING - STEP + u < nj) issue(j0 + RING - STEP + u);
    tile_scores(j0);
    if constexpr (STEP == 2)
      if (j0 + 1 < nj) tile_scores(j0 + 1);
  }
  if (a.write_masked && active && blockIdx.y == 0)
    for (int s = p + 1 + lane; s < a.Lk; s += 64) out[s] = kNegInf;
}

int pick_ksplit(int blocks, int ntiles_max) {
  int ks = 1;
  while (blocks * ks < 1024 && ks * 8 <= ntiles_max) ks *= 2;
  return ks;
}

template <bool FP8>
hipError_t launch_mfma(const IndexLaunch& a, hipStream_t s) {
  if (a.q_count <= kDecodeIndexQueries) {
    static_assert(kDecChunk == kCandChunk, "candidate lists follow the work-group chunks");
    if (a.cand_m && (a.cand_m > kCandCap || (a.cand_m & 7) || !a.cand_keys || !a.cand_offs || !a.cand_hdr))
      return hipErrorInvalidValue;
    dim3 grid((a.Lk + kDecChunk - 1) / kDecChunk, a.B * a.q_count);
    launch_kernel(idx_decode_kernel<FP8>, grid, dim3(256), 0, s, a);
  } else {
    // only the decode kernel clears zero_hist and writes candidate lists
    if (a.zero_hist || a.cand_m) return hipErrorInvalidValue;
    constexpr int QB = 8;
    const int nqb = (a.q_count + QB - 1) / QB;
    const int n_max = a.Lk - a.Lq + a.q_begin + a.q_count;
    const int ks = pick_ksplit(nqb * a.B, (n_max + 63) / 64);
    dim3 grid(nqb, ks, a.B);
    launch_kernel(idx_prefill_kernel<FP8, QB>, grid, dim3(QB * 64), 0, s, a, ks);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_index_f32(const IndexLaunch& a, hipStream_t s) {
  if (a.zero_hist || a.cand_m) return hipErrorInvalidValue;   // decode kernel only
  dim3 grid((a.Lk + 255) / 256, a.B * a.q_count);
  const size_t smem = (size_t)(a.H * a.D + a.H) * sizeof(float);
  launch_kernel(idx_f32_kernel, grid, dim3(256), smem, s, a);
  return hipGetLastError();
}

hipError_t launch_index_bf16(const IndexLaunch& a, hipStream_t s) { return launch_mfma<false>(a, s); }
hipError_t launch_index_fp8(const IndexLaunch& a, hipStream_t s) { return launch_mfma<true>(a, s); }

}  // namespace dsa
