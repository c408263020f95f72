// Sparse MLA attention (absorbed MQA form) over the selected latent rows.
//
// For query (b, i), head a and the chosen positions S:
//     z_j  = scale * q_a . kv_j                    (kv_j: 576 = 512 latent + 64 rope)
//     out_a = sum_{j in S} softmax_j(z) * kv_j[0:512]
//     lse_a = log sum_j exp(z_j)
// HF model doc "DeepSeek-V3.2", section "DeepSeek Sparse Attention (DSA)",
// item 2 (attention over the chosen tokens only); altools.ai "Technical
// Principles" (MLA in MQA form: one cached entry per token serves all query
// heads); dims from the released configuration excerpt on the atlas
// "DeepSeek-V3.2-Exp" token-ids page (n_heads 128, kv_lora_rank 512,
// qk_rope_head_dim 64).
//
// bf16 kernel, one work-group per (query, key split), 8 waves x 16 heads:
//  - the selected rows are gathered from HBM in blocks of 32 straight into
//    LDS (global_load_lds: each lane moves one 16-byte chunk of a 1152-byte
//    row, no registers involved), three blocks in flight, and staged once
//    for all 128 heads;
//  - S^T = KV_blk . Q^T on 16x16x32 MFMA (Q stays in registers), so each
//    lane column owns one head and the softmax max/sum are lane-local plus
//    two cross-lane exchanges;
//  - online softmax in base 2, with the running max only raised when a block
//    exceeds it by more than 2^8 (the accumulator rescale is then rare);
//  - O^T += V^T . P^T on MFMA with P taken straight from the S^T registers
//    and the value operand read transposed from the row-major tile
//    (ds_read_b64_tr_b16), so no second copy of the values is staged.
// Decode-shaped launches split each query's list over several work-groups
// and merge the partial (O, lse) pairs in a second kernel.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr float kNegInf = -__builtin_inff();
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ------------------------------------------------------------- bf16 -------
constexpr int kNH = 128, kDqk = 576, kDv = 512, kBK = 32;
constexpr int kRowB = kDqk * 2;                 // 1152 bytes per kv row = 72 chunks of 16 B
constexpr int kChunks = kRowB / 16;
constexpr int kStageBytes = kBK * kRowB;        // one 32-row block in LDS
constexpr int kMaxPer = 4096;                   // list entries per work-group
constexpr float kTau = 8.0f;                    // lazy max threshold (log2 units)

#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))
#define GLB_PTR(p) ((const __attribute__((address_space(1))) void*)(p))
typedef short i16x4 __attribute__((ext_vector_type(4)));

// Rows of a staged block sit back to back (1152 B = 8 bank quads mod 16);
// the 16-byte chunk c of row r is stored at chunk c ^ swz(r), which keeps
// both the 16-row MFMA operand reads (one chunk of 16 consecutive rows) and
// the transposed value reads (two chunks of 4 rows) on distinct bank quads.
__device__ __forceinline__ int swz(int r) {
  const int j = (r >> 1) & 7;
  return (j >> 1) | ((j & 1) << 2);
}

// s_waitcnt on the vector-memory counter only (gfx9 encoding: expcnt and
// lgkmcnt fields left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | (((N >> 4) & 3) << 14));
}

// 16-byte global -> LDS copy per lane (LDS destination = lds_base + 16*lane).
// Written as asm so that the compiler's wait-count pass does not treat the
// in-flight copies into other stage buffers as hazards for the current one;
// completion is awaited explicitly with wait_vmcnt<>().  The instruction has
// no register outputs.
// M0 is reserved by the compiler (gfx9 LDS instructions do not read it and
// nothing else in these kernels uses it); it is named as clobbered anyway.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* gbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_base), "v"(voff), "s"(gbase)
               : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)(p);
}

__device__ __forceinline__ u32x2 tr_read(const uint8_t* p) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// Work split: 8 waves x 16 heads.  Per wave and 32-key block, on 16x16x32
// MFMA: S^T (2 key tiles x 16 heads, 18 k-steps over 576 dims) and
// O^T (32 value tiles x 16 heads, one k-step over the 32 keys).
// Lane l: column = head 16*wave + (l % 16), k-group g = l / 16.
//   S^T rows (keys) held: 4g + i and 16 + 4g + i, i = 0..3.
//   O^T rows (value dims) held: 16*vt + 4g + i.
constexpr int kWavesA = 8;
constexpr int kQRegSteps = 16;                  // k-steps of Q kept in registers (latent dims)
struct AttnState {
  u32x4 qf[kQRegSteps];  // Q^T fragments (B operand): dims 32t + 8g .. +8 of this lane's head
  f32x4 o[32];         // O^T accumulators
  float m_run, l_run;
};

// Gather instructions per wave per block: 36 x 64-lane 16-byte copies
// split 5,5,5,5,4,4,4,4 over the 8 waves.
__device__ __forceinline__ int dma_first(int wave) { return wave < 4 ? 5 * wave : 20 + 4 * (wave - 4); }

// One 32-row block: S^T = KV.Q^T, online softmax, O^T += V^T.P^T.
__device__ __forceinline__ void attn_block(AttnState& st, const uint8_t* buf, const int* bpos,
                                           const uint8_t* qrope, const int (&qk_off)[2][2],
                                           const int (&pv_off)[2][4], int g, float zscale) {
  f32x4 s[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) s[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < 18; ++t) {
    const u32x4 qb = t < kQRegSteps ? st.qf[t < kQRegSteps ? t : 0] : ld16(qrope + 64 * (t - kQRegSteps));
#pragma unroll
    for (int m = 0; m < 2; ++m)
      s[m] = mfma16(ld16(buf + qk_off[m][t & 1] + 128 * (t >> 1)), qb, s[m]);
  }
  float z[8];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const u32x4 pv = *reinterpret_cast<const u32x4*>(bpos + 16 * m + 4 * g);
#pragma unroll
    for (int r = 0; r < 4; ++r) z[4 * m + r] = ((int)pv[r] >= 0) ? s[m][r] * zscale : kNegInf;
  }
  float mb = z[0];
#pragma unroll
  for (int e = 1; e < 8; ++e) mb = fmaxf(mb, z[e]);
  mb = fmaxf(mb, shfl_xor(mb, 16));
  mb = fmaxf(mb, shfl_xor(mb, 32));
  if (__ballot(mb > st.m_run + kTau)) {
    const float m_new = fmaxf(st.m_run, mb);
    const float alpha = (st.m_run == kNegInf) ? 0.f : exp2f(st.m_run - m_new);
#pragma unroll
    for (int v = 0; v < 32; ++v) st.o[v] *= alpha;
    st.l_run *= alpha;
    st.m_run = m_new;
  }
  const float mref = (st.m_run == kNegInf) ? 0.f : st.m_run;
  u32x4 pb;
  float lsum = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t u = pack_bf16x2(exp2f(z[2 * e] - mref), exp2f(z[2 * e + 1] - mref));
    pb[e] = u;
    lsum += bf16_lo(u) + bf16_hi(u);
  }
  st.l_run += lsum;
#pragma unroll
  for (int vt = 0; vt < 32; ++vt) {
    const int imm = 128 * (vt >> 2);
    const u32x2 lo = tr_read(buf + pv_off[0][vt & 3] + imm);
    const u32x2 hi = tr_read(buf + pv_off[1][vt & 3] + imm);
    const u32x4 av = {lo[0], lo[1], hi[0], hi[1]};
    st.o[vt] = mfma16(av, pb, st.o[vt]);
  }
}

__global__ __launch_bounds__(kWavesA * 64, 1) void attn_bf16_kernel(AttnLaunch a) {
  __shared__ __attribute__((aligned(16))) uint8_t stg[3 * kStageBytes];
  __shared__ __attribute__((aligned(16))) int spos[kMaxPer];
  __shared__ __attribute__((aligned(16))) uint8_t qrope_s[kNH * 128];   // rope dims of Q, per head
  __shared__ int s_last;

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c16 = lane & 15;
  const int split = blockIdx.x;
  const int rr = gridDim.y - 1 - blockIdx.y;    // launch row; latest queries first
  const int b = rr / a.q_count;
  const int i = a.q_begin + rr % a.q_count;
  const int64_t qrow = (int64_t)b * a.Lq + i;
  const int per = ((a.K + a.splits - 1) / a.splits + kBK - 1) / kBK * kBK;
  const int j0 = split * per;
  const int nent = max(0, min(a.K, j0 + per) - j0);

  // Chosen positions of this split into LDS (-1 for skipped / padding).
  if (tid == 0) s_last = -1;
  __syncthreads();
  int my_last = -1;
  const int32_t* idx = a.idx + qrow * a.K + j0;
  for (int j = tid; j < per; j += kWavesA * 64) {
    int pos = j < nent ? idx[j] : -1;
    if (pos >= a.Lk) pos = -1;
    spos[j] = pos < 0 ? -1 : pos;
    if (pos >= 0) my_last = j;
  }
  if (my_last >= 0) atomicMax(&s_last, my_last);

  AttnState st;
  const int h = 16 * wave + c16;
  {
    const uint8_t* qb = static_cast<const uint8_t*>(a.qa) + (qrow * kNH + h) * (int64_t)kRowB;
#pragma unroll
    for (int t = 0; t < kQRegSteps; ++t) st.qf[t] = ld16(qb + (32 * t + 8 * g) * 2);
    // rope k-steps: head h's 64 dims (8 chunks) at qrope_s + 128h; this
    // lane's chunk for k-step 16 + u is 4u + g
#pragma unroll
    for (int u = 0; u < 18 - kQRegSteps; ++u)
      st16(qrope_s + 128 * h + 16 * (4 * u + g), ld16(qb + (32 * (kQRegSteps + u) + 8 * g) * 2));
  }
#pragma unroll
  for (int v = 0; v < 32; ++v) st.o[v] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.m_run = kNegInf;
  st.l_run = 0.f;
  const float zscale = a.scale * kLog2e;

  // QK operand: key row 16m + c16, logical chunk 4t + g, stored at
  // (4t + g) ^ swz(row) = 4 * (t ^ (y >> 2)) + (y & 3) with y = g ^ swz(row).
  int qk_off[2][2];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int row = 16 * m + c16;
    const int y = g ^ swz(row);
    const int base = row * kRowB + 16 * (y & 3);
    const int flip = (y >> 2) ? 64 : 0;
    qk_off[m][0] = base + flip;                    // even t: 64t = 128(t>>1)
    qk_off[m][1] = base + 64 - flip;               // odd t:  64t = 128(t>>1) + 64
  }
  // PV operand (transposed reads): group g = lane/16 takes keys 4g + e
  // (first read) and 16 + 4g + e (second); source lane j = lane%16 reads
  // row key0 + j/4, value columns 16vt + 4(j&3) .. +3, i.e. logical chunk
  // 2vt + ((j&3) >> 1), half (j & 1).  Stored chunk (2vt + x) ^ swz(row)
  // = 2 * (vt ^ (y >> 1)) + (y & 1), y = x ^ swz(row).
  int pv_off[2][4];
  {
    const int x = (c16 & 3) >> 1, within = (c16 & 1) * 8;
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const int row = 16 * w + 4 * g + (c16 >> 2);
      const int y = x ^ swz(row);
#pragma unroll
      for (int k = 0; k < 4; ++k) pv_off[w][k] = row * kRowB + 16 * (y & 1) + within + 32 * (k ^ (y >> 1));
    }
  }
  __syncthreads();
  const int nblk = (s_last + kBK) / kBK;          // blocks up to the last listed entry

  // Gather map: instruction k of this wave fills LDS chunk slots
  // f = (dma_first(wave) + k)*64 + lane: row f/72, stored chunk f%72, which
  // holds logical chunk (f%72) ^ swz(row).
  const int dfirst = dma_first(wave);
  const int dcount = wave < 4 ? 5 : 4;
  const uint8_t* kvb = static_cast<const uint8_t*>(a.kv) + (int64_t)b * a.Lk * kRowB;   // uniform
  const uint32_t stg_lds = lds_addr(stg);
  auto issue = [&](int blk, int sb) {
    const uint32_t dst = __builtin_amdgcn_readfirstlane(stg_lds + sb * kStageBytes);
#pragma unroll
    for (int k = 0; k < 5; ++k) {
      if (k < dcount) {
        const int f = (dfirst + k) * 64 + lane;
        const int r = f / kChunks, p = f - r * kChunks;
        const int pos = max(spos[blk * kBK + r], 0);
        dma16(kvb, (uint32_t)pos * kRowB + ((p ^ swz(r)) << 4),
              __builtin_amdgcn_readfirstlane(dst + (dfirst + k) * 1024));
      }
    }
  };
  // Block blk lives in stage buffer blk % 3.  Wait for its gather (the next
  // block's may stay in flight), barrier (every wave is then also done with
  // block blk-1's buffer), start the gather two blocks ahead into that
  // buffer, then compute.
  if (nblk > 0) issue(0, 0);
  if (nblk > 1) issue(1, 1);
  int sb = 0;
  for (int blk = 0; blk < nblk; ++blk) {
    if (blk + 1 < nblk) {
      if (dcount == 5) wait_vmcnt<5>();
      else wait_vmcnt<4>();
    } else {
      wait_vmcnt<0>();
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);           // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (blk + 2 < nblk) issue(blk + 2, sb == 0 ? 2 : sb - 1);
    attn_block(st, stg + sb * kStageBytes, spos + blk * kBK, qrope_s + 128 * h + 16 * g, qk_off, pv_off, g,
               zscale);
    sb = sb == 2 ? 0 : sb + 1;
  }

  float l_tot = st.l_run + shfl_xor(st.l_run, 16);
  l_tot += shfl_xor(l_tot, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse = l_tot > 0.f ? (st.m_run + log2f(l_tot)) * kLn2 : kNegInf;
  if (a.splits == 1) {
    if (a.out_f32) {
      float* op = static_cast<float*>(a.out) + (qrow * kNH + h) * kDv + 4 * g;
#pragma unroll
      for (int vt = 0; vt < 32; ++vt) *reinterpret_cast<f32x4*>(op + 16 * vt) = st.o[vt] * inv;
    } else {
      uint16_t* op = static_cast<uint16_t*>(a.out) + (qrow * kNH + h) * kDv + 4 * g;
#pragma unroll
      for (int vt = 0; vt < 32; ++vt) {
        const f32x4 v = st.o[vt] * inv;
        *reinterpret_cast<u32x2*>(op + 16 * vt) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      }
    }
    if (a.lse && g == 0) a.lse[qrow * kNH + h] = lse;
  } else {
    const int64_t prow = (int64_t)rr * a.splits + split;
    float* op = a.part_o + (prow * kNH + h) * kDv + 4 * g;
#pragma unroll
    for (int vt = 0; vt < 32; ++vt) *reinterpret_cast<f32x4*>(op + 16 * vt) = st.o[vt] * inv;
    if (g == 0) a.part_lse[prow * kNH + h] = lse;
  }
}

// Merge split partials: out = sum_s exp(lse_s - LSE) * O_s, LSE = log sum_s exp(lse_s).
// grid (NH, rows), Dv/4 threads.
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnLaunch a) {
  const int h = blockIdx.x, rr = blockIdx.y, v = threadIdx.x * 4;
  const int S = a.splits, NH = a.NH, Dv = a.Dv;
  const int b = rr / a.q_count;
  const int i = a.q_begin + rr % a.q_count;
  const int64_t qrow = (int64_t)b * a.Lq + i;
  const float* pl = a.part_lse + (int64_t)rr * S * NH + h;
  float m = kNegInf;
  for (int s = 0; s < S; ++s) m = fmaxf(m, pl[(int64_t)s * NH]);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float sum = 0.f;
  if (m != kNegInf) {
    for (int s = 0; s < S; ++s) {
      const float ls = pl[(int64_t)s * NH];
      if (ls == kNegInf) continue;
      const float wgt = __expf(ls - m);
      sum += wgt;
      const f32x4 po = *reinterpret_cast<const f32x4*>(a.part_o + (((int64_t)rr * S + s) * NH + h) * Dv + v);
      acc += wgt * po;
    }
    acc *= 1.f / sum;
  }
  if (v < Dv) {
    if (a.out_f32) {
      *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + (qrow * NH + h) * Dv + v) = acc;
    } else {
      u32x2 v2 = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
      *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.out) + (qrow * NH + h) * Dv + v) = v2;
    }
  }
  if (a.lse && threadIdx.x == 0) a.lse[qrow * NH + h] = m == kNegInf ? kNegInf : m + __logf(sum);
}

// ------------------------------------------------------------- fp32 -------
// One work-group per (query, head): logits for every listed key into LDS,
// max / sum by block reduction, then each thread owns value dims.
__global__ __launch_bounds__(256) void attn_f32_kernel(AttnLaunch a) {
  extern __shared__ float sm[];
  const int Dqk = a.Dqk, Dv = a.Dv, K = a.K, NH = a.NH;
  float* qs = sm;                 // Dqk
  float* zs = sm + Dqk;           // K
  __shared__ float red[8];
  const int h = blockIdx.x, rr = blockIdx.y, tid = threadIdx.x;
  const int b = rr / a.q_count;
  const int i = a.q_begin + rr % a.q_count;
  const int64_t qrow = (int64_t)b * a.Lq + i;
  const float* qg = static_cast<const float*>(a.qa) + (qrow * NH + h) * Dqk;
  const float* kvb = static_cast<const float*>(a.kv) + (int64_t)b * a.Lk * Dqk;
  const int32_t* idx = a.idx + qrow * K;
  for (int d = tid; d < Dqk; d += 256) qs[d] = qg[d];
  __syncthreads();
  float mloc = kNegInf;
  for (int j = tid; j < K; j += 256) {
    const int pos = idx[j];
    float z = kNegInf;
    if (pos >= 0 && pos < a.Lk) {
      const float* r = kvb + (int64_t)pos * Dqk;
      float acc = 0.f;
      for (int d = 0; d < Dqk; ++d) acc = fmaf(qs[d], r[d], acc);
      z = acc * a.scale;
    }
    zs[j] = z;
    mloc = fmaxf(mloc, z);
  }
  mloc = wave_max(mloc);
  if ((tid & 63) == 0) red[tid >> 6] = mloc;
  __syncthreads();
  const float m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  float sloc = 0.f;
  for (int j = tid; j < K; j += 256) {
    const float p = zs[j] == kNegInf ? 0.f : __expf(zs[j] - m);
    zs[j] = p;
    sloc += p;
  }
  sloc = wave_sum(sloc);
  if ((tid & 63) == 0) red[4 + (tid >> 6)] = sloc;
  __syncthreads();
  const float l = red[4] + red[5] + red[6] + red[7];
  const float inv = l > 0.f ? 1.f / l : 0.f;
  float* op = static_cast<float*>(a.out) + (qrow * NH + h) * Dv;
  for (int v = tid; v < Dv; v += 256) {
    float acc = 0.f;
    for (int j = 0; j < K; ++j) {
      const int pos = idx[j];
      if (pos >= 0 && pos < a.Lk) acc = fmaf(zs[j], kvb[(int64_t)pos * Dqk + v], acc);
    }
    op[v] = acc * inv;
  }
  if (a.lse && tid == 0) a.lse[qrow * NH + h] = l > 0.f ? m + __logf(l) : kNegInf;
}

}  // namespace

int attn_splits_bf16(int rows, int K) {
  const int max_splits = (K + 63) / 64;           // at least 64 keys per split
  int s = 1;
  while (rows * s < 256 && s * 2 <= max_splits) s *= 2;
  // a split's list window lives in LDS: at most kMaxPer entries
  while (((K + s - 1) / s + kBK - 1) / kBK * kBK > kMaxPer) s *= 2;
  return s;
}

hipError_t launch_attn_bf16(const AttnLaunch& a, hipStream_t s) {
  dim3 grid(a.splits, a.B * a.q_count);
  hipLaunchKernelGGL(attn_bf16_kernel, grid, dim3(kWavesA * 64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_attn_combine(const AttnLaunch& a, hipStream_t s) {
  dim3 grid(a.NH, a.B * a.q_count);
  hipLaunchKernelGGL(attn_combine_kernel, grid, dim3(a.Dv / 4), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_attn_f32(const AttnLaunch& a, hipStream_t s) {
  dim3 grid(a.NH, a.B * a.q_count);
  const size_t smem = (size_t)(a.Dqk + a.K) * sizeof(float);
  hipLaunchKernelGGL(attn_f32_kernel, grid, dim3(256), smem, s, a);
  return hipGetLastError();
}

}  // namespace dsa
