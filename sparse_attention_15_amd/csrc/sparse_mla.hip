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
// bf16 kernel, one work-group per (query, key split), 4 waves of 32 heads:
//  - the selected rows are gathered from HBM in blocks of 32 straight into
//    LDS (global_load_lds: each lane moves one 16-byte chunk of a 1152-byte
//    row, no registers involved), three stage buffers with two blocks in
//    flight, and staged once for all 128 heads; the next-but-one block's
//    gather is issued from inside the current block's QK steps;
//  - S^T = KV_blk . Q^T on 32x32x16 MFMA over all 576 dims, Q in registers
//    (each wave's 32 head rows staged once through LDS); each lane owns one
//    head, so the softmax max/sum are lane-local plus one cross-half
//    exchange;
//  - online softmax in base 2 with the logit scale folded into the exponent's
//    FMA, the running max only raised when a block exceeds it by more than
//    2^8 (the accumulator rescale is then rare);
//  - O^T += V^T . P^T on MFMA with P taken straight from the S^T registers
//    and the value operand read transposed from the row-major tile
//    (ds_read_b64_tr_b16), so no second copy of the values is staged; the
//    second key half's P is formed while the first half's PV MFMAs run;
//  - output rows leave through the idle stage buffers, 1 KB contiguous per
//    store instruction.
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
// Decode split partials in fp32 for bf16 outputs too (one output rounding
// instead of two).  Off: it doubles the partial bytes, +8.4 us per 32 x 32K
// decode step (attention +3.7, combine +4.3) and +2.7 us at 8 x 128K, while
// the second rounding stays far inside the bf16 output tolerance.
constexpr bool kF32Partials = false;

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

// 16-byte global -> LDS copy per lane (LDS destination = lds_base + 16*lane,
// global source = gbase + row_off + (map >> 8)).  Written as asm so that the
// compiler's wait-count pass does not treat the in-flight copies into other
// stage buffers as hazards for the current one; completion is awaited
// explicitly with wait_vmcnt<>().  The address add sits inside the asm so
// that the LDS read of row_off is only waited for here.  No memory clobber:
// the copies only target a stage buffer that nothing reads before the next
// barrier, and the asm stays ordered after that barrier (both are volatile
// asm).  An SALU write of M0 needs one wait state before an LDS-DMA reads it.
// M0 is named as clobbered (nothing else in these kernels uses it).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* gbase, uint32_t row_off, uint32_t map, uint32_t lds_base) {
  uint32_t t;
  asm volatile(
      "v_lshrrev_b32 %0, 8, %2\n\t"
      "v_add_u32 %0, %0, %1\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %4"
      : "=&v"(t)
      : "v"(row_off), "v"(map), "s"(lds_base), "s"(gbase)
      : "m0");
}
#pragma clang diagnostic pop

// max over lanes l and l ^ 32 (v_permlane32_swap, no LDS round trip)
__device__ __forceinline__ float max_xor32(float x) {
  float a, b;
  xor32_pair(x, a, b);
  return fmaxf(a, b);
}

__device__ __forceinline__ u32x2 tr_read(const uint8_t* p) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// Work split: 4 waves, one per SIMD, so each wave has the whole register
// file of its SIMD (512 registers: the O accumulators live in AGPRs).  Wave w
// owns heads 32w .. 32w+31 for all 576 dims and all 512 value dims, on
// 32x32x16 MFMA, so no partial scores cross waves.
// Lane l: column = head 32w + (l % 32), half hf = l / 32.
//   S^T rows (keys) held: 8q + 4hf + r, q, r = 0..3.
//   O^T rows (value dims) held: 32vt + 8q + 4hf + r, vt = 0..15.
constexpr int kWavesA = 4;
constexpr int kQSteps = kDqk / 16;               // 36 k-steps of 16 dims
constexpr int kVTiles = kDv / 32;                // 16 value tiles of 32 dims
struct AttnState {
  u32x4 qf[kQSteps];   // Q^T fragments (B operand)
  f32x16 o[kVTiles];   // O^T accumulators
  float m_run, l_run;
};

// Gather instructions per wave per block: 38 x 64-lane 16-byte copies
// split 10, 10, 9, 9 over the 4 waves.
constexpr int kDmaMax = 10;
__device__ __forceinline__ int dma_first(int wave) { return wave < 2 ? 10 * wave : 20 + 9 * (wave - 2); }
static_assert(kDmaInstr == 38, "gather split assumes 38 instructions per block");

// QK MFMAs with the accumulator in VGPRs.  The kernel's builtin MFMAs (PV)
// are selected in AGPR form, which puts the 256-register O accumulator in the
// AGPR file; writing the QK chain as asm keeps S (and Q) in VGPRs instead of
// a second AGPR tile.  Back-to-back accumulation into the same registers
// needs no wait states; the last step of the chain waits out the result
// latency before any VALU instruction reads S (24 wait states, more than the
// 8-pass MFMA needs).
__device__ __forceinline__ void qk_first(f32x16& d, const u32x4& a, const u32x4& b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void qk_next(f32x16& d, const u32x4& a, const u32x4& b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void qk_last(f32x16& d, const u32x4& a, const u32x4& b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(d) : "v"(a), "v"(b));
}

__device__ __forceinline__ void scale_tile(f32x16& o, float alpha) {
  float e[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) e[k] = o[k];
  float t;
  asm volatile(
      "s_nop 7\n\ts_nop 7\n\ts_nop 7\n\t"
#define R(k) "v_accvgpr_read_b32 %16, %" #k "\n\tv_mul_f32 %16, %17, %16\n\tv_accvgpr_write_b32 %" #k ", %16\n\t"
      R(0) R(1) R(2) R(3) R(4) R(5) R(6) R(7) R(8) R(9) R(10) R(11) R(12) R(13) R(14) R(15)
#undef R
      "s_nop 4"
      : "+a"(e[0]), "+a"(e[1]), "+a"(e[2]), "+a"(e[3]), "+a"(e[4]), "+a"(e[5]), "+a"(e[6]), "+a"(e[7]),
        "+a"(e[8]), "+a"(e[9]), "+a"(e[10]), "+a"(e[11]), "+a"(e[12]), "+a"(e[13]), "+a"(e[14]), "+a"(e[15]),
        "=&v"(t)
      : "v"(alpha));
#pragma unroll
  for (int k = 0; k < 16; ++k) o[k] = e[k];
}

// Row gathers of a later block, issued from inside the QK chain of the
// current one so that their address and issue latency overlaps the MFMAs.
struct Gather {
  const uint8_t* kvb;     // this sequence's latent rows (wave-uniform)
  const uint32_t* bp;     // LDS row byte offsets of the block to gather
  uint32_t dst;           // LDS stage buffer of that block
  int dfirst, dcount;     // this wave's gather instructions
  bool active;            // wave-uniform: is there a block to gather
};

// One 32-row block.
__device__ __forceinline__ void attn_block(AttnState& st, const uint8_t* buf, uint32_t vmask,
                                           const int (&qk_off)[2], const int (&pv_off)[2][2], int hf,
                                           float zscale, const Gather& g, const uint32_t (&dma_map)[kDmaMax]) {
  // gather instruction k: its row positions are read from LDS after QK step
  // 3k - 1 and the copy is issued after step 3k + 1, so the LDS latency
  // of the position read hides behind two MFMAs
  // gather instruction k: the row's byte offset is read from LDS after QK
  // step 3k - 1 and the copy is issued after step 3k + 1
  uint32_t roff[kDmaMax];
  auto addr = [&](int k) {
    uint32_t m = dma_map[k];
    asm("" : "+v"(m));                          // keep the packed form (one register)
    roff[k] = g.bp[m & 0xffu];
  };
  if (g.active) addr(0);
  // A operands: a ring of kRing LDS reads in flight ahead of the MFMAs
  constexpr int kRing = 4;
  u32x4 av[kRing];
#pragma unroll
  for (int t = 0; t < kRing; ++t) av[t] = ld16(buf + qk_off[t & 1] + 64 * (t >> 1));
  f32x16 s;
#pragma unroll
  for (int t = 0; t < kQSteps; ++t) {
    const u32x4 a_t = av[t % kRing];
    if (t + kRing < kQSteps) av[t % kRing] = ld16(buf + qk_off[(t + kRing) & 1] + 64 * ((t + kRing) >> 1));
    if (t == 0) qk_first(s, a_t, st.qf[t]);
    else if (t == kQSteps - 1) qk_last(s, a_t, st.qf[t]);
    else qk_next(s, a_t, st.qf[t]);
    if (t % 3 == 2 && t / 3 + 1 < kDmaMax) {
      const int k = t / 3 + 1;
      if (g.active && k < g.dcount) addr(k);
    }
    if (t % 3 == 1 && t / 3 < kDmaMax) {
      const int k = t / 3;
      if (g.active && k < g.dcount)
        dma16(g.kvb, roff[k], dma_map[k], __builtin_amdgcn_readfirstlane(g.dst + (g.dfirst + k) * 1024));
    }
  }
  // base-2 logits z = zscale * s.  With zscale > 0 (the usual case) the scale
  // is folded into the exponent's FMA and the max is taken on raw scores;
  // otherwise the scores are scaled first.  Keys not listed in this block
  // (bit clear in vmask) get -inf.  This lane's keys: 8q + 4hf + r.
  float fs = zscale;
  if (!(zscale > 0.f)) {
#pragma unroll
    for (int e = 0; e < 16; ++e) s[e] *= zscale;
    fs = 1.f;
  }
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
  mb = max_xor32(mb) * fs;
  if (__ballot(mb > st.m_run + kTau)) {
    const float m_new = fmaxf(st.m_run, mb);
    if (__ballot(st.m_run != kNegInf)) {          // before the first raise O and l are zero
      const float alpha = (st.m_run == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(st.m_run - m_new);
#pragma unroll
      for (int v = 0; v < kVTiles; ++v) scale_tile(st.o[v], alpha);
      st.l_run *= alpha;
    }
    st.m_run = m_new;
  }
  const float nref = (st.m_run == kNegInf) ? 0.f : -st.m_run;
  // p = 2^(z - m) <= 2^kTau; P is rounded to bf16 for the MFMA, the
  // normaliser sums the fp32 values (the rounding is unbiased and far below
  // the output rounding).  The two 16-key halves of P feed the two PV k-steps,
  // so the second half's exponentials can overlap the first half's MFMAs.
  float lsum = 0.f;
  // O^T[v][head] += V^T[v][key] . P^T[key][head]
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    u32x4 pb;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float p0 = __builtin_amdgcn_exp2f(fmaf(s[8 * k + 2 * e], fs, nref));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(s[8 * k + 2 * e + 1], fs, nref));
      pb[e] = pack_bf16x2(p0, p1);
      lsum += p0 + p1;
    }
#pragma unroll
    for (int vt = 0; vt < kVTiles; ++vt) {
      const u32x2 lo = tr_read(buf + pv_off[k][0] + 64 * vt);
      const u32x2 hi = tr_read(buf + pv_off[k][1] + 64 * vt);
      const u32x4 av = {lo[0], lo[1], hi[0], hi[1]};
      st.o[vt] = mfma32(av, pb, st.o[vt]);
    }
  }
  st.l_run += lsum;
}

// NST stage buffers (NST - 1 blocks in flight) and a list window of MAXPER
// entries.  LDS holds 3 buffers next to a 2048-entry window, or 4 next to a
// 256-entry one: decode splits have short windows and their gathers are
// random HBM rows, so they keep one more block in flight, and every wave
// stages its Q rows at once.
template <int NST, int MAXPER>
__global__ __launch_bounds__(kWavesA * 64, 1) void attn_bf16_kernel(AttnLaunch a) {
  static_assert((NST == 3 || NST == 4) && MAXPER % (kWavesA * 64) == 0, "stage / window shape");
  __shared__ __attribute__((aligned(16))) uint8_t stg[NST * kStageBytes];
  __shared__ __attribute__((aligned(16))) uint32_t spos[MAXPER];
  __shared__ uint32_t bmask[MAXPER / kBK];        // per 32-entry block: bit j = entry j usable
  __shared__ int s_lastw[kWavesA];

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = lane >> 5, c32 = lane & 31;
  int split = blockIdx.x;
  int rr = gridDim.y - 1 - blockIdx.y;          // launch row; latest queries first
  if (a.splits > 1 && (gridDim.y & 7) == 0) {
    // Work-groups are dealt to the 8 XCDs round-robin by linear id, so ids
    // x, x+8, x+16, ... share an L2: give them all splits of rows x, x+8, ...
    // (the splits of a query then fetch its Q rows into one L2 once).
    const int lin = blockIdx.x + gridDim.x * blockIdx.y;
    const int loc = lin >> 3;
    rr = (lin & 7) + 8 * (loc / a.splits);
    split = loc - (loc / a.splits) * a.splits;
  }
  const int b = rr / a.q_count;
  const int i = a.q_begin + rr % a.q_count;
  const int64_t qrow = (int64_t)b * a.Lq + i;
  const int per = ((a.K + a.splits - 1) / a.splits + kBK - 1) / kBK * kBK;
  const int j0 = split * per;
  const int nent = max(0, min(a.K, j0 + per) - j0);

  // This split's list entries (all loads in flight at once), then the Q rows
  // of this wave's 32 heads staged in a stage buffer (read back with the key
  // rows' conflict-free addressing).  Four buffers: every wave now, into its
  // own buffer.  Three: waves 0-2 now into buffers 0-2 by LDS-DMA (whole
  // cache lines), wave 3 after the first barrier into buffer 2, while blocks
  // 0 and 1 are gathered into buffers 0 and 1.
  constexpr int kFillIt = MAXPER / (kWavesA * 64);
  int pv[kFillIt];
  const int32_t* idx = a.idx + qrow * a.K + j0;
#pragma unroll
  for (int it = 0; it < kFillIt; ++it) {
    const int j = (it * kWavesA + wave) * 64 + lane;
    pv[it] = j < nent ? idx[j] : -1;
  }
  AttnState st;
  const int h = 32 * wave + c32;
  const uint8_t* qwave = static_cast<const uint8_t*>(a.qa) + (qrow * kNH + 32 * wave) * (int64_t)kRowB;  // uniform
  const uint32_t stg_lds = lds_addr(stg);
  auto gather_q = [&](int buf) {
    const uint32_t dst = __builtin_amdgcn_readfirstlane(stg_lds + buf * kStageBytes);
#pragma unroll 2
    for (int k = 0; k < kDmaInstr; ++k) {
      const int f = k * 64 + lane;
      const int r = f / kLdsChunks, p = f - r * kLdsChunks;
      const uint32_t off = (uint32_t)r * kRowB + (p < kChunks ? (uint32_t)((p ^ swz(r)) << 4) : 0u);
      lds_dma16<false>(qwave, off, dst + k * 1024);
    }
  };
  // Four buffers (decode splits): every wave loads its 36 KB of Q rows into
  // registers with coalesced 16-byte loads, all in flight at once, and
  // writes them to its buffer below (LDS-DMA copies would queue behind the
  // few a wave keeps in flight).
  if (NST == 4) {
    const u32x4* qsrc = reinterpret_cast<const u32x4*>(qwave);
#pragma unroll
    for (int k = 0; k < kQSteps; ++k) st.qf[k] = qsrc[k * 64 + lane];
  } else if (wave < 3) {
    gather_q(wave);
  }
  // Chosen rows into LDS as byte offsets (row * 1152; skipped and padding
  // entries point at row 0), one validity bit per entry in bmask (bit j of
  // word w: entry 32w + j is usable), and each wave's last usable entry.
  int my_last = -1;
#pragma unroll
  for (int it = 0; it < kFillIt; ++it) {
    const int jw = (it * kWavesA + wave) * 64;
    if (jw < per) {
      int pos = pv[it];
      if (pos >= a.Lk) pos = -1;
      const uint64_t bal = __ballot(pos >= 0);
      spos[jw + lane] = (uint32_t)max(pos, 0) * kRowB;
      if (lane == 0) {
        bmask[jw / kBK] = (uint32_t)bal;
        if (jw + kBK < per) bmask[jw / kBK + 1] = (uint32_t)(bal >> 32);
      }
      if (bal) my_last = jw + 63 - __builtin_clzll(bal);
    }
  }
  if (lane == 0) s_lastw[wave] = my_last;

#pragma unroll
  for (int v = 0; v < kVTiles; ++v)
#pragma unroll
    for (int e = 0; e < 16; ++e) st.o[v][e] = 0.f;
  st.m_run = kNegInf;
  st.l_run = 0.f;
  const float zscale = a.scale * kLog2e;

  // QK operand: key row c32, logical chunk 2t + hf
  //   = 4(t >> 1) + (2(t & 1) + hf), stored with the low two bits
  //   XOR swz(row): offset qk_off[t & 1] + 64 * (t >> 1).
  int qk_off[2];
  {
    const int f = swz(c32);
#pragma unroll
    for (int par = 0; par < 2; ++par) qk_off[par] = c32 * kLdsRow + 16 * ((2 * par + hf) ^ f);
  }
  auto read_q = [&](int buf) {
    const uint8_t* qbuf = stg + buf * kStageBytes;
#pragma unroll
    for (int t = 0; t < kQSteps; ++t) st.qf[t] = ld16(qbuf + qk_off[t & 1] + 64 * (t >> 1));
  };
  if (NST == 4) {
    // register k of lane l holds 16-byte chunk 64k + l of the wave's rows:
    // row f / 72, chunk f % 72, stored at the chunk's permuted slot
    uint8_t* qbuf = stg + wave * kStageBytes;
#pragma unroll
    for (int k = 0; k < kQSteps; ++k) {
      const int f = k * 64 + lane;
      const int r = f / kChunks, c = f - r * kChunks;
      *reinterpret_cast<u32x4*>(qbuf + r * kLdsRow + 16 * (c ^ swz(r))) = st.qf[k];
    }
    read_q(wave);
  } else if (wave < 3) {
    wait_vmcnt<0>();                              // this wave's Q rows have landed
    read_q(wave);
  }
  // PV operand (transposed reads) for 32x32x16: 16-lane group G holds value
  // rows 16(G&1) + j of the tile and k-half G>>1.  Step k, part w (lo/hi)
  // reads key row 16k + 8w + 4(G>>1) + j/4, value columns
  // 32vt + 16(G&1) + 4(j&3) .. +3: logical chunk 4vt + k0 with
  // k0 = 2(G&1) + (j&3)/2, byte (j&1)*8; stored at 4vt + (k0 ^ swz):
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
        pv_off[k][w] = row * kLdsRow + 16 * (k0 ^ swz(row)) + within;
      }
  }
  __syncthreads();
  const int last = max(max(s_lastw[0], s_lastw[1]), max(s_lastw[2], s_lastw[3]));
  const int nblk = (last + kBK) / kBK;            // blocks up to the last listed entry
  if (NST == 3 && wave == 3) gather_q(2);        // wave 2 has read its Q from buffer 2

  // Gather map: instruction k of this wave fills LDS chunk slots
  // f = (dma_first(wave) + k)*64 + lane: row f/76, stored chunk f%76, which
  // holds logical chunk (f%76) ^ swz(row).  Slots 72..75 of a row are
  // padding that no operand read touches; their lanes copy the row's first
  // chunk there (same cache line as a real copy), so every lane of a gather
  // instruction is active and the addressing has no branches.
  const int dfirst = dma_first(wave);
  const int dcount = wave < 2 ? 10 : 9;
  // per lane and gather instruction: row (low 8 bits) | global byte offset
  // within the row << 8
  uint32_t dma_map[kDmaMax];
#pragma unroll
  for (int k = 0; k < kDmaMax; ++k) {
    const int f = (dfirst + k) * 64 + lane;
    const int r = f / kLdsChunks, p = f - r * kLdsChunks;
    dma_map[k] = k >= dcount ? 0u : ((uint32_t)r | ((uint32_t)(p < kChunks ? (p ^ swz(r)) << 4 : 0) << 8));
  }
  const uint8_t* kvb = static_cast<const uint8_t*>(a.kv) + (int64_t)b * a.Lc * kRowB;   // uniform
  auto issue = [&](int blk, int sb) {
    const uint32_t dst = __builtin_amdgcn_readfirstlane(stg_lds + sb * kStageBytes);
    const uint32_t* bp = spos + blk * kBK;
    uint32_t roff[kDmaMax];
#pragma unroll
    for (int k = 0; k < kDmaMax; ++k) roff[k] = bp[dma_map[k] & 0xffu];
#pragma unroll
    for (int k = 0; k < kDmaMax; ++k)
      if (k < dcount) dma16(kvb, roff[k], dma_map[k], __builtin_amdgcn_readfirstlane(dst + (dfirst + k) * 1024));
  };
  // Block blk lives in stage buffer blk % NST.  Wait for its gather (later
  // blocks' may stay in flight) and barrier: every wave is then also done
  // with block blk-1, whose buffer receives block blk+NST-1, gathered from
  // inside block blk's QK steps.
#pragma unroll
  for (int j = 0; j < NST - 1; ++j)
    if (nblk > j) issue(j, j);
  if (NST == 3 && wave == 3) {                    // Q rows are older than the block gathers
    if (nblk > 1) wait_vmcnt<18>();
    else if (nblk > 0) wait_vmcnt<9>();
    else wait_vmcnt<0>();
    read_q(2);
  }
  // Consume the Q fragments here so that their LDS reads are complete before
  // the loop (with three buffers, block 2 is gathered into buffer 2, wave
  // 3's Q staging, during block 0).
#pragma unroll
  for (int t = 0; t < kQSteps; ++t) asm volatile("" : "+v"(st.qf[t]));
  int sb = 0;
  Gather g;
  g.kvb = kvb;
  g.dfirst = dfirst;
  g.dcount = dcount;
  for (int blk = 0; blk < nblk; ++blk) {
    // block blk has landed once at most `ahead` later blocks are in flight
    const int ahead = min(nblk - 1 - blk, NST - 2);
    if (ahead == 2) {
      if (dcount == 10) wait_vmcnt<20>();
      else wait_vmcnt<18>();
    } else if (ahead == 1) {
      if (dcount == 10) wait_vmcnt<10>();
      else wait_vmcnt<9>();
    } else {
      wait_vmcnt<0>();
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);           // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    const int sn = sb == 0 ? NST - 1 : sb - 1;     // buffer of blocks blk-1 and blk+NST-1
    g.active = blk + NST - 1 < nblk;
    g.bp = spos + (blk + NST - 1) * kBK;
    g.dst = __builtin_amdgcn_readfirstlane(stg_lds + sn * kStageBytes);
    const uint32_t vmask = __builtin_amdgcn_readfirstlane(bmask[blk]);
    attn_block(st, stg + sb * kStageBytes, vmask, qk_off, pv_off, hf, zscale, g, dma_map);
    sb = sb == NST - 1 ? 0 : sb + 1;
  }

  const float l_tot = st.l_run + shfl_xor(st.l_run, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse = l_tot > 0.f ? (st.m_run + log2f(l_tot)) * kLn2 : kNegInf;

  const bool f32 = a.out_f32 != 0;
  if (a.splits > 1) {
    const bool pf32 = kF32Partials || f32;
    // A split's partial leaves straight from the accumulators in their
    // register order (no LDS round trip, no barrier): for value tile vt and
    // quad q the wave stores its 64 lanes' four values contiguously, 512
    // bytes (bf16) or 1 KB (fp32) per instruction.  Value r of lane l in
    // block (wave w, vt, q) is O[head 32w + l % 32][dim 32vt + 8q + 4(l / 32) + r];
    // attn_combine_kernel reads this layout.
    const int64_t prow = (int64_t)rr * a.splits + split;
    if (hf == 0) a.part_lse[prow * kNH + h] = lse;
    const int64_t blk0 = (prow * kWavesA + wave) * kVTiles * 4;   // this wave's first (vt, q) block
    if (pf32) {
      f32x4* dst = static_cast<f32x4*>(a.part_o) + blk0 * 64 + lane;
#pragma unroll
      for (int vt = 0; vt < kVTiles; ++vt)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          dst[(vt * 4 + q) * 64] = f32x4{st.o[vt][4 * q] * inv, st.o[vt][4 * q + 1] * inv,
                                         st.o[vt][4 * q + 2] * inv, st.o[vt][4 * q + 3] * inv};
    } else {
      u32x2* dst = static_cast<u32x2*>(a.part_o) + blk0 * 64 + lane;
#pragma unroll
      for (int vt = 0; vt < kVTiles; ++vt)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          dst[(vt * 4 + q) * 64] = u32x2{pack_bf16x2(st.o[vt][4 * q] * inv, st.o[vt][4 * q + 1] * inv),
                                         pack_bf16x2(st.o[vt][4 * q + 2] * inv, st.o[vt][4 * q + 3] * inv)};
    }
    return;
  }

  // Output rows through LDS: per pass the wave writes a slice of its 32 head
  // rows (512 bytes each) into the now idle stage buffers, then stores 1 KB
  // contiguous per instruction (two 512-byte row segments) instead of 16
  // bytes into each of 32 rows.
  __syncthreads();                                // every wave is done with the stage buffers
  uint8_t* dst_base = static_cast<uint8_t*>(a.out) + (qrow * kNH + 32 * wave) * (int64_t)kDv * (f32 ? 4 : 2);
  if (a.lse && hf == 0) a.lse[qrow * kNH + h] = lse;
  constexpr int kEpiRow = 528;                    // 512 bytes + 16 bytes of padding per head row
  uint8_t* ebuf = stg + wave * 32 * kEpiRow;
  const int row_bytes = kDv * (f32 ? 4 : 2);
  auto flush = [&](int pass) {                    // ebuf rows -> bytes [512 pass, +512) of each head row
    __builtin_amdgcn_s_waitcnt(0xc07f);           // lgkmcnt(0): this wave's LDS writes are done
#pragma unroll
    for (int it = 0; it < 16; ++it) {
      const int r = 2 * it + (lane >> 5);
      const u32x4 v = ld16(ebuf + r * kEpiRow + 16 * (lane & 31));
      st16(dst_base + (int64_t)r * row_bytes + 512 * pass + 16 * (lane & 31), v);
    }
  };
  if (f32) {
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {        // 4 value tiles (128 dims) per pass
#pragma unroll
      for (int vt = 4 * pass; vt < 4 * pass + 4; ++vt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 v4 = {st.o[vt][4 * q] * inv, st.o[vt][4 * q + 1] * inv, st.o[vt][4 * q + 2] * inv,
                            st.o[vt][4 * q + 3] * inv};
          *reinterpret_cast<f32x4*>(ebuf + c32 * kEpiRow + ((vt - 4 * pass) * 32 + 8 * q + 4 * hf) * 4) = v4;
        }
      flush(pass);
    }
  } else {
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {        // 8 value tiles (256 dims) per pass
#pragma unroll
      for (int vt = 8 * pass; vt < 8 * pass + 8; ++vt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const u32x2 v2 = {pack_bf16x2(st.o[vt][4 * q] * inv, st.o[vt][4 * q + 1] * inv),
                            pack_bf16x2(st.o[vt][4 * q + 2] * inv, st.o[vt][4 * q + 3] * inv)};
          *reinterpret_cast<u32x2*>(ebuf + c32 * kEpiRow + ((vt - 8 * pass) * 32 + 8 * q + 4 * hf) * 2) = v2;
        }
      flush(pass);
    }
  }
}

// Merge split partials: out = sum_s exp(lse_s - LSE) * O_s, LSE = log sum_s exp(lse_s).
// The partials are in the attention kernel's register order (see its
// epilogue).  grid (4 * 16 / VT, rows): work-group x covers heads 32w ..
// 32w+31 (w = x / (16 / VT)) and VT value tiles from VT vg (vg = x % (16 /
// VT)), i.e. 32 VT dims: a 2 VT KB (bf16) or 4 VT KB (fp32) block of each
// split's partial.  Thread t takes that block's 16-byte-aligned pair of
// lanes 2t, 2t+1 (two heads, four dims each), loads it for G splits at a
// time (all in flight together), adds the splits in order with fp32
// weights and stores its two 4-dim pieces.  The 32 heads' weights come from
// their LSEs while the partials load.  Few rows take VT = 1 (twice the
// work-groups, every split in flight at once for bf16).
template <int S, bool F32, int VT>
__global__ __launch_bounds__(128 * VT) void attn_combine_kernel(AttnLaunch a) {
  constexpr bool PF32 = kF32Partials || F32;      // partial precision
  constexpr int EB = PF32 ? 4 : 2;                // bytes per partial value
  constexpr int OB = F32 ? 4 : 2;                 // bytes per output value
  constexpr int LD = 2 * 4 * EB / 16;             // 16-byte loads per thread and split
  constexpr int GM = VT == 1 ? (PF32 ? 16 : 32) : (PF32 ? 8 : 16);
  constexpr int G = GM < S ? GM : S;              // splits in flight at once
  constexpr int NVG = kVTiles / VT;               // work-groups per 32 heads
  __shared__ float wt[S][32];
  int gx = blockIdx.x, rr = blockIdx.y;
  if ((gridDim.y & 7) == 0) {                     // row rr on the XCD its splits ran on
    const int lin = blockIdx.x + gridDim.x * blockIdx.y;
    const int loc = lin >> 3;
    rr = (lin & 7) + 8 * (loc / gridDim.x);
    gx = loc - (loc / gridDim.x) * gridDim.x;
  }
  const int w = gx / NVG, vg = gx - w * NVG, tid = threadIdx.x;
  const int NH = a.NH;
  const int b = rr / a.q_count;
  const int i = a.q_begin + rr % a.q_count;
  const int64_t qrow = (int64_t)b * a.Lq + i;
  // this thread's lanes l0, l0+1 of block (w, vt, q) of every split
  const int c = 2 * tid;                          // chunk within the 512 chunks of (w, vg)
  const int vt = VT * vg + (c >> 8), q = (c >> 6) & 3, l0 = c & 63;
  const int64_t split_u4 = (int64_t)NH * a.Dv * EB / 16;          // 16-byte units per split
  const u32x4* src = static_cast<const u32x4*>(a.part_o) + (int64_t)rr * S * split_u4 +
                     ((((int64_t)w * kVTiles + vt) * 4 + q) * 64 + l0) * (4 * EB) / 16;
  u32x4 v[G][LD];
#pragma unroll
  for (int s = 0; s < G; ++s)
#pragma unroll
    for (int k = 0; k < LD; ++k) v[s][k] = src[s * split_u4 + k];
  if (tid < 32) {
    const int h = 32 * w + tid;
    const float* pl = a.part_lse + (int64_t)rr * S * NH + h;
    float m = kNegInf;
#pragma unroll
    for (int s = 0; s < S; ++s) m = fmaxf(m, pl[(int64_t)s * NH]);
    float sum = 0.f;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const float ls = pl[(int64_t)s * NH];
      const float e = (m == kNegInf || ls == kNegInf) ? 0.f : __expf(ls - m);   // an empty split holds zeros
      wt[s][tid] = e;
      sum += e;
    }
    const float inv = sum > 0.f ? 1.f / sum : 0.f;
#pragma unroll
    for (int s = 0; s < S; ++s) wt[s][tid] *= inv;
    if (a.lse && vg == 0) a.lse[qrow * NH + h] = m == kNegInf ? kNegInf : m + __logf(sum);
  }
  __syncthreads();
  const int hl = l0 & 31, hf = l0 >> 5;           // heads hl, hl+1; dims 32vt + 8q + 4hf + r
  float acc[2][4];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[j][r] = 0.f;
  auto add = [&](int s0) {
#pragma unroll
    for (int s = 0; s < G; ++s) {
      float x[8];                                 // lane l0 + j, value r at 4j + r
      if constexpr (PF32) {
#pragma unroll
        for (int k = 0; k < LD; ++k) {
          const f32x4 f = __builtin_bit_cast(f32x4, v[s][k]);
#pragma unroll
          for (int e = 0; e < 4; ++e) x[4 * k + e] = f[e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[2 * e] = bf16_lo(v[s][0][e]);
          x[2 * e + 1] = bf16_hi(v[s][0][e]);
        }
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float wj = wt[s0 + s][hl + j];
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[j][r] += wj * x[4 * j + r];
      }
    }
  };
  add(0);
#pragma unroll
  for (int s0 = G; s0 < S; s0 += G) {
#pragma unroll
    for (int s = 0; s < G; ++s)
#pragma unroll
      for (int k = 0; k < LD; ++k) v[s][k] = src[(s0 + s) * split_u4 + k];
    add(s0);
  }
  // out[head 32w + hl + j][dims 32vt + 8q + 4hf .. +3]: per store
  // instruction the wave's 64 pieces land as 64-byte runs of 16 head rows
  const int d0 = 32 * vt + 8 * q + 4 * hf;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    uint8_t* o = static_cast<uint8_t*>(a.out) + ((qrow * NH + 32 * w + hl + j) * (int64_t)a.Dv + d0) * OB;
    if constexpr (F32) {
      *reinterpret_cast<f32x4*>(o) = f32x4{acc[j][0], acc[j][1], acc[j][2], acc[j][3]};
    } else {
      *reinterpret_cast<u32x2*>(o) = u32x2{pack_bf16x2(acc[j][0], acc[j][1]), pack_bf16x2(acc[j][2], acc[j][3])};
    }
  }
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
  const float* kvb = static_cast<const float*>(a.kv) + (int64_t)b * a.Lc * Dqk;
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

constexpr int kCombFewRows = 16;

int attn_splits_bf16(int rows, int K) {
  // at least 128 keys (4 blocks) per split: a split's fixed costs (list, Q,
  // first gathers, epilogue) and its 128 KB of partials for the combine
  // outweigh the work of fewer keys (8 queries of 2048 keys: 32 splits of
  // 64 keys 31.5 us attention + combine, 16 of 128 keys 29.3 us, 8 of 256
  // keys 32.9 us)
  const int max_splits = (K + 127) / 128;
  int s = 1;
  while (rows * s < 256 && s * 2 <= max_splits && s < 32) s *= 2;
  // a split's list window lives in LDS: at most kMaxPer entries (K <= 65536
  // keeps this at 32 splits or fewer, the combine kernel's largest variant)
  while (((K + s - 1) / s + kBK - 1) / kBK * kBK > kMaxPer) s *= 2;
  return s;
}

hipError_t launch_attn_bf16(const AttnLaunch& a, hipStream_t s) {
  dim3 grid(a.splits, a.B * a.q_count);
  const int per = ((a.K + a.splits - 1) / a.splits + kBK - 1) / kBK * kBK;
  if (per <= 256)
    launch_kernel(attn_bf16_kernel<4, 256>, grid, dim3(kWavesA * 64), 0, s, a);
  else
    launch_kernel(attn_bf16_kernel<3, kMaxPer>, grid, dim3(kWavesA * 64), 0, s, a);
  return hipGetLastError();
}

template <bool F32, int VT>
hipError_t launch_combine_vt(const AttnLaunch& a, hipStream_t s) {
  dim3 grid(4 * (kVTiles / VT), a.B * a.q_count);
  dim3 block(128 * VT);
  switch (a.splits) {
    case 2: launch_kernel(attn_combine_kernel<2, F32, VT>, grid, block, 0, s, a); break;
    case 4: launch_kernel(attn_combine_kernel<4, F32, VT>, grid, block, 0, s, a); break;
    case 8: launch_kernel(attn_combine_kernel<8, F32, VT>, grid, block, 0, s, a); break;
    case 16: launch_kernel(attn_combine_kernel<16, F32, VT>, grid, block, 0, s, a); break;
    case 32: launch_kernel(attn_combine_kernel<32, F32, VT>, grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;       // splits are powers of two up to 32
  }
  return hipGetLastError();
}

template <bool F32>
hipError_t launch_combine_t(const AttnLaunch& a, hipStream_t s) {
  // fewer than 16 rows: 64 work-groups per row instead of 32
  return a.B * a.q_count < kCombFewRows ? launch_combine_vt<F32, 1>(a, s) : launch_combine_vt<F32, 2>(a, s);
}

// bf16 kernel shapes only: NH = 128, Dv = 512 (the attention kernel's register order)
hipError_t launch_attn_combine(const AttnLaunch& a, hipStream_t s) {
  if (a.NH != kNH || a.Dv != kDv) return hipErrorInvalidValue;
  return a.out_f32 ? launch_combine_t<true>(a, s) : launch_combine_t<false>(a, s);
}

hipError_t launch_attn_f32(const AttnLaunch& a, hipStream_t s) {
  dim3 grid(a.NH, a.B * a.q_count);
  const size_t smem = (size_t)(a.Dqk + a.K) * sizeof(float);
  launch_kernel(attn_f32_kernel, grid, dim3(256), smem, s, a);
  return hipGetLastError();
}

}  // namespace dsa
