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
// bf16 kernel, one work-group per (query, key split), 8 waves in 4 pairs:
//  - the selected rows are gathered from HBM in blocks of 32 straight into
//    LDS (global_load_lds: each lane moves one 16-byte chunk of a 1152-byte
//    row, no registers involved), three blocks in flight, and staged once
//    for all 128 heads;
//  - S^T = KV_blk . Q^T on 32x32x16 MFMA, the 576 dims split between the two
//    waves of a pair and the partial tiles summed through LDS (Q stays in
//    registers); each lane owns one head, so the softmax max/sum are
//    lane-local plus one cross-half exchange;
//  - online softmax in base 2, with the running max only raised when a block
//    exceeds it by more than 2^8 (the accumulator rescale is then rare);
//  - O^T += V^T . P^T on MFMA with P taken straight from the S^T registers
//    and the value operand read transposed from the row-major tile
//    (ds_read_b64_tr_b16), so no second copy of the values is staged; the
//    two partners cover the two halves of the 512 value dims.
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
constexpr int kLdsChunks = 76;                  // LDS row stride in 16-byte chunks (4 unused)
constexpr int kLdsRow = kLdsChunks * 16;
constexpr int kStageBytes = kBK * kLdsRow;      // one 32-row block in LDS
constexpr int kDmaInstr = kBK * kLdsChunks / 64;  // 38 gather instructions per block
constexpr int kMaxPer = 2048;                   // list entries per work-group
constexpr float kTau = 8.0f;                    // lazy max threshold (log2 units)

#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))
#define GLB_PTR(p) ((const __attribute__((address_space(1))) void*)(p))
typedef short i16x4 __attribute__((ext_vector_type(4)));

// A staged block holds 32 rows of 76 16-byte chunks (72 used).  The row
// stride and the chunk permutation (chunk c of row r stored at c ^ swz(r),
// swz(r) < 4, i.e. within aligned groups of four) were chosen by measuring
// both operand read patterns on gfx950: they spread the rows of a 32-row QK
// operand read and the 8-row transposed value reads over the LDS banks, and
// keep every operand address a per-lane base plus a compile-time offset.
__device__ __forceinline__ int swz(int r) { return ((r >> 2) + 1) & 3; }

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

// max over lanes l and l ^ 32 (v_permlane32_swap exchanges the two halves
// of the wave without going through LDS)
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x),
                                                  false, false);
  return fmaxf(__builtin_bit_cast(float, r[0]), __builtin_bit_cast(float, r[1]));
}

__device__ __forceinline__ u32x2 tr_read(const uint8_t* p) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// Work split: 8 waves = 4 pairs; pair p owns heads 32p .. 32p+31 and the two
// partners split the work, per 32-key block, on 32x32x16 MFMA:
//   QK: partner d computes the partial S^T over dims [288d, 288d + 288)
//       (18 k-steps; its Q^T fragments stay in 72 registers), writes it to
//       LDS, and after a barrier adds the other partner's partial, so both
//       hold the same full S^T (fp32 addition commutes);
//   softmax: done identically by both partners;
//   PV: partner d accumulates O^T for value dims [256d, 256d + 256).
// Lane l: column = head 32p + (l % 32), half hf = l / 32.
//   S^T rows (keys) held: 8q + 4hf + r, q, r = 0..3.
//   O^T rows (value dims) held: 256d + 32vt + 8q + 4hf + r.
constexpr int kWavesA = 8;
constexpr int kQSteps = 18;                      // 16-dim k-steps per partner
constexpr int kVTiles = 8;                       // 32-wide value tiles per partner
struct AttnState {
  u32x4 qf[kQSteps];   // Q^T fragments (B operand)
  f32x16 o[kVTiles];   // O^T accumulators
  float m_run, l_run;
};

// Gather instructions per wave per block: 38 x 64-lane 16-byte copies
// split 5,5,5,5,5,5,4,4 over the 8 waves.
__device__ __forceinline__ int dma_first(int wave) { return wave < 6 ? 5 * wave : 30 + 4 * (wave - 6); }
static_assert(kDmaInstr == 38, "gather split assumes 38 instructions per block");

// One 32-row block.
__device__ __forceinline__ void attn_block(AttnState& st, const uint8_t* buf, uint32_t vmask, float* exch_mine,
                                           const float* exch_other, const int (&qk_off)[2],
                                           const int (&pv_off)[2][2], int hf, float zscale) {
  f32x16 s;
#pragma unroll
  for (int e = 0; e < 16; ++e) s[e] = 0.f;
#pragma unroll
  for (int t = 0; t < kQSteps; ++t) s = mfma32(ld16(buf + qk_off[t & 1] + 64 * (t >> 1)), st.qf[t], s);
  // exchange partial scores with the partner wave (lane-linear, 4 x 16 B)
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const f32x4 v = {s[4 * q], s[4 * q + 1], s[4 * q + 2], s[4 * q + 3]};
    *reinterpret_cast<f32x4*>(exch_mine + q * 256) = v;
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);             // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(exch_other + q * 256);
    s[4 * q] += v[0];
    s[4 * q + 1] += v[1];
    s[4 * q + 2] += v[2];
    s[4 * q + 3] += v[3];
  }
  // scaled base-2 logits; keys not listed in this block (bit clear in
  // vmask) get -inf.  This lane's keys: 8q + 4hf + r.
#pragma unroll
  for (int e = 0; e < 16; ++e) s[e] *= zscale;
  if (vmask != 0xffffffffu) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int key = 8 * (e >> 2) + 4 * hf + (e & 3);
      s[e] = ((vmask >> key) & 1u) ? s[e] : kNegInf;
    }
  }
  float mb = fmaxf(fmaxf(s[0], s[1]), s[2]);
#pragma unroll
  for (int e = 3; e < 15; e += 2) mb = fmaxf(fmaxf(mb, s[e]), s[e + 1]);
  mb = fmaxf(mb, s[15]);
  mb = max_xor32(mb);
  if (__ballot(mb > st.m_run + kTau)) {
    const float m_new = fmaxf(st.m_run, mb);
    const float alpha = (st.m_run == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(st.m_run - m_new);
#pragma unroll
    for (int v = 0; v < kVTiles; ++v) st.o[v] *= alpha;
    st.l_run *= alpha;
    st.m_run = m_new;
  }
  const float mref = (st.m_run == kNegInf) ? 0.f : st.m_run;
  // p = 2^(z - m) <= 2^kTau; P is rounded to bf16 for the MFMA, the
  // normaliser sums the fp32 values (the rounding is unbiased and far below
  // the output rounding)
  u32x4 pb[2];
  float lsum = 0.f;
#pragma unroll
  for (int k = 0; k < 2; ++k)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float p0 = __builtin_amdgcn_exp2f(s[8 * k + 2 * e] - mref);
      const float p1 = __builtin_amdgcn_exp2f(s[8 * k + 2 * e + 1] - mref);
      pb[k][e] = pack_bf16x2(p0, p1);
      lsum += p0 + p1;
    }
  st.l_run += lsum;
  // O^T[v][head] += V^T[v][key] . P^T[key][head]
#pragma unroll
  for (int vt = 0; vt < kVTiles; ++vt)
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const u32x2 lo = tr_read(buf + pv_off[k][0] + 64 * vt);
      const u32x2 hi = tr_read(buf + pv_off[k][1] + 64 * vt);
      const u32x4 av = {lo[0], lo[1], hi[0], hi[1]};
      st.o[vt] = mfma32(av, pb[k], st.o[vt]);
    }
}

__global__ __launch_bounds__(kWavesA * 64, 1) void attn_bf16_kernel(AttnLaunch a) {
  __shared__ __attribute__((aligned(16))) uint8_t stg[3 * kStageBytes];
  __shared__ __attribute__((aligned(16))) int spos[kMaxPer];
  __shared__ uint32_t bmask[kMaxPer / kBK];       // per 32-entry block: bit j = entry j usable
  __shared__ __attribute__((aligned(16))) float exch[kWavesA * 1024];   // 4 KiB of partial scores per wave
  __shared__ int s_last;

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = lane >> 5, c32 = lane & 31;
  const int pair = wave >> 1, d = wave & 1;
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
  const int h = 32 * pair + c32;
  {
    const uint8_t* qb = static_cast<const uint8_t*>(a.qa) + (qrow * kNH + h) * (int64_t)kRowB + 576 * d;
#pragma unroll
    for (int t = 0; t < kQSteps; ++t) st.qf[t] = ld16(qb + (16 * t + 8 * hf) * 2);
  }
#pragma unroll
  for (int v = 0; v < kVTiles; ++v)
#pragma unroll
    for (int e = 0; e < 16; ++e) st.o[v][e] = 0.f;
  st.m_run = kNegInf;
  st.l_run = 0.f;
  const float zscale = a.scale * kLog2e;

  // QK operand: key row c32, logical chunk 36d + 2t + hf
  //   = 36d + 4(t >> 1) + (2(t & 1) + hf), stored with the low two bits
  //   XOR swz(row): offset qk_off[t & 1] + 64 * (t >> 1).
  int qk_off[2];
  {
    const int f = swz(c32);
#pragma unroll
    for (int par = 0; par < 2; ++par) qk_off[par] = c32 * kLdsRow + 576 * d + 16 * ((2 * par + hf) ^ f);
  }
  // PV operand (transposed reads) for 32x32x16: 16-lane group G holds value
  // rows 16(G&1) + j of the tile and k-half G>>1.  Step k, part w (lo/hi)
  // reads key row 16k + 8w + 4(G>>1) + j/4, value columns
  // 256d + 32vt + 16(G&1) + 4(j&3) .. +3: logical chunk 32d + 4vt + k0 with
  // k0 = 2(G&1) + (j&3)/2, byte (j&1)*8; stored at 32d + 4vt + (k0 ^ swz):
  // offset pv_off[k][w] + 64 * vt.
  int pv_off[2][2];
  {
    const int G = lane >> 4, j = lane & 15;
    const int k0 = 2 * (G & 1) + ((j & 3) >> 1), within = (j & 1) * 8;
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const int row = 16 * k + 8 * w + 4 * (G >> 1) + (j >> 2);
        pv_off[k][w] = row * kLdsRow + 16 * (32 * d + (k0 ^ swz(row))) + within;
      }
  }
  __syncthreads();
  const int nblk = (s_last + kBK) / kBK;          // blocks up to the last listed entry
  // Consume the Q fragments here so that their loads are complete before the
  // loop: the compiler's own vector-memory waits would otherwise stay inside
  // the loop and also stall on the in-flight row gathers.
#pragma unroll
  for (int t = 0; t < kQSteps; ++t) asm volatile("" : "+v"(st.qf[t]));
  for (int blk = wave; blk < nblk; blk += kWavesA) {
    const uint64_t bal = __ballot(lane < kBK && spos[blk * kBK + (lane & (kBK - 1))] >= 0);
    if (lane == 0) bmask[blk] = (uint32_t)bal;
  }
  __syncthreads();

  // Gather map: instruction k of this wave fills LDS chunk slots
  // f = (dma_first(wave) + k)*64 + lane: row f/76, stored chunk f%76 (slots
  // 72..75 are padding and stay unloaded), which holds logical chunk
  // (f%76) ^ swz(row).
  const int dfirst = dma_first(wave);
  const int dcount = wave < 6 ? 5 : 4;
  // per lane and gather instruction: row (low 8 bits) | stored-chunk byte
  // offset << 8, or ~0u for a padding slot
  uint32_t dma_map[5];
#pragma unroll
  for (int k = 0; k < 5; ++k) {
    const int f = (dfirst + k) * 64 + lane;
    const int r = f / kLdsChunks, p = f - r * kLdsChunks;
    dma_map[k] = p < kChunks ? ((uint32_t)r | ((uint32_t)((p ^ swz(r)) << 4) << 8)) : ~0u;
  }
  const uint8_t* kvb = static_cast<const uint8_t*>(a.kv) + (int64_t)b * a.Lk * kRowB;   // uniform
  const uint32_t stg_lds = lds_addr(stg);
  auto issue = [&](int blk, int sb) {
    const uint32_t dst = __builtin_amdgcn_readfirstlane(stg_lds + sb * kStageBytes);
    const int* bp = spos + blk * kBK;
    uint32_t voff[5];
#pragma unroll
    for (int k = 0; k < 5; ++k) {               // all position reads first: one LDS latency
      uint32_t m = dma_map[k];
      asm volatile("" : "+v"(m));               // keep the packed form (one register)
      voff[k] = m == ~0u ? ~0u : (uint32_t)max(bp[m & 0xffu], 0) * kRowB + (m >> 8);
    }
#pragma unroll
    for (int k = 0; k < 5; ++k) {
      if (k < dcount) {
        const uint32_t ldst = __builtin_amdgcn_readfirstlane(dst + (dfirst + k) * 1024);
        if (voff[k] != ~0u) dma16(kvb, voff[k], ldst);
      }
    }
  };
  float* exch_mine = exch + wave * 1024 + lane * 4;
  const float* exch_other = exch + (wave ^ 1) * 1024 + lane * 4;
  // Block blk lives in stage buffer blk % 3.  Wait for its gather (the next
  // block's may stay in flight), barrier (every wave is then also done with
  // block blk-1's buffer and scores exchange), start the gather two blocks
  // ahead into that buffer, then compute.
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
    const uint32_t vmask = __builtin_amdgcn_readfirstlane(bmask[blk]);
    attn_block(st, stg + sb * kStageBytes, vmask, exch_mine, exch_other, qk_off, pv_off, hf, zscale);
    sb = sb == 2 ? 0 : sb + 1;
  }

  const float l_tot = st.l_run + shfl_xor(st.l_run, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse = l_tot > 0.f ? (st.m_run + log2f(l_tot)) * kLn2 : kNegInf;
  const int vbase = 256 * d + 4 * hf;
  if (a.splits == 1) {
    if (a.out_f32) {
      float* op = static_cast<float*>(a.out) + (qrow * kNH + h) * kDv + vbase;
#pragma unroll
      for (int vt = 0; vt < kVTiles; ++vt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 v4 = {st.o[vt][4 * q] * inv, st.o[vt][4 * q + 1] * inv, st.o[vt][4 * q + 2] * inv,
                            st.o[vt][4 * q + 3] * inv};
          *reinterpret_cast<f32x4*>(op + 32 * vt + 8 * q) = v4;
        }
    } else {
      uint16_t* op = static_cast<uint16_t*>(a.out) + (qrow * kNH + h) * kDv + vbase;
#pragma unroll
      for (int vt = 0; vt < kVTiles; ++vt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const u32x2 v2 = {pack_bf16x2(st.o[vt][4 * q] * inv, st.o[vt][4 * q + 1] * inv),
                            pack_bf16x2(st.o[vt][4 * q + 2] * inv, st.o[vt][4 * q + 3] * inv)};
          *reinterpret_cast<u32x2*>(op + 32 * vt + 8 * q) = v2;
        }
    }
    if (a.lse && hf == 0 && d == 0) a.lse[qrow * kNH + h] = lse;
  } else {
    const int64_t prow = (int64_t)rr * a.splits + split;
    float* op = a.part_o + (prow * kNH + h) * kDv + vbase;
#pragma unroll
    for (int vt = 0; vt < kVTiles; ++vt)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 v4 = {st.o[vt][4 * q] * inv, st.o[vt][4 * q + 1] * inv, st.o[vt][4 * q + 2] * inv,
                          st.o[vt][4 * q + 3] * inv};
        *reinterpret_cast<f32x4*>(op + 32 * vt + 8 * q) = v4;
      }
    if (hf == 0 && d == 0) a.part_lse[prow * kNH + h] = lse;
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
