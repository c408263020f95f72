// Exact per-row top-k on gfx950.
//
// Each query keeps the index_topk best-scoring positions (HF model doc
// "DeepSeek-V3.2", section "DeepSeek Sparse Attention (DSA)", item 2; a query
// with fewer candidates takes all of them, visual-learn "DeepSeek-V3.2 / Exp",
// "Different questions select different tokens").  Order: larger score first,
// lower position first among equal scores; +0.0 and -0.0 are equal.  Output:
// the chosen positions ascending, padded with -1.
//
// One work-group per row.  Scores become order-preserving 32-bit keys; an
// MSB-first radix select (12 + 12 + 8 bits, LDS histograms) finds the
// threshold key T and how many elements equal to T are still needed (r).
// The selection is then {key > T} plus the first r positions with key == T,
// and one ordered pass writes it: for a chosen element at position x its
// output slot is  #(key > T before x) + min(#(key == T before x), r),
// so block-wide scans of packed (gt, eq) counts give the slots (DPP wave
// scans, one barrier per group of 8 chunks).
// Row values stay in registers (4 consecutive positions per 16-byte load);
// rows longer than the register budget are re-read from memory each pass.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;

__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  if (u == 0x80000000u) u = 0u;                 // -0.0 == +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// DPP source shift (lanes whose source is out of range read 0).
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWS, 0xf, false);
}

// Inclusive scan over the 64 lanes: shifts by 1, 2, 4, 8 within each row of
// 16 lanes, then row 0's total into row 1 and row 2's into row 3
// (row_bcast:15), then lane 31's running total into rows 2 and 3
// (row_bcast:31).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v, int) {
  v += dpp<0x111, 0xf>(v);
  v += dpp<0x112, 0xf>(v);
  v += dpp<0x114, 0xf>(v);
  v += dpp<0x118, 0xf>(v);
  v += dpp<0x142, 0xa>(v);
  v += dpp<0x143, 0xc>(v);
  return v;
}

constexpr int kGroup = 8;            // chunks per emission group

struct Shared {
  uint32_t hist[4096];
  uint32_t wsum[kGroup * kWaves];
  uint32_t bin;        // chosen bin of the current pass
  uint32_t above;      // elements in bins above it
};

// Find the bin holding the k-th largest element (k >= 1) of hist[0..nb).
// Thread t owns a run of bins counted from the top, so a block-wide scan of
// the per-thread sums gives each run the number of elements above it.
// Returns via sh.bin / sh.above.  All threads must call.
__device__ void find_bin(Shared& sh, int nb, uint32_t k) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int per = nb >= kThreads ? nb / kThreads : 1;
  const int hi = nb - per * tid;                 // my bins: [hi - per, hi)
  uint32_t local = 0;
  if (hi > 0)
    for (int j = 1; j <= per; ++j) local += sh.hist[hi - j];
  const uint32_t incl = wave_incl_scan(local, lane);
  if (lane == 63) sh.wsum[wave] = incl;
  __syncthreads();
  uint32_t before = 0;
  for (int w = 0; w < wave; ++w) before += sh.wsum[w];
  uint32_t run = before + incl - local;          // count strictly above my bins
  if (run < k && run + local >= k) {
    for (int j = 1; j <= per; ++j) {
      const uint32_t c = sh.hist[hi - j];
      if (run + c >= k) {
        sh.bin = hi - j;
        sh.above = run;
        break;
      }
      run += c;
    }
  }
  __syncthreads();
}

template <int NC>  // NC 16-byte chunks per thread kept in registers; 0 = stream
__global__ __launch_bounds__(kThreads) void topk_kernel(TopkLaunch a) {
  __shared__ Shared sh;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = gridDim.x - 1 - blockIdx.x;     // longest rows first
  const int b = row / a.q_count;
  const int i = a.q_begin + row % a.q_count;
  const int n = a.Lk - a.Lq + i + 1;
  const int K = a.K;
  int32_t* out = a.out + ((int64_t)b * a.Lq + i) * K;
  const float* src = a.scores + (int64_t)row * a.row_stride;

  if (n <= K) {
    for (int j = tid; j < K; j += kThreads) out[j] = j < n ? j : -1;
    return;
  }
  const int nchunks = (n + 3) >> 2;               // 4 positions per chunk
  const int iters = (nchunks + kThreads - 1) / kThreads;

  auto load_keys = [&](int c, uint32_t (&kk)[4]) {
    const int ch = c * kThreads + tid;
    const int pos = ch * 4;
    if (a.vec_ok && pos + 3 < n) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(src + pos);
      kk[0] = order_key(v.x);
      kk[1] = order_key(v.y);
      kk[2] = order_key(v.z);
      kk[3] = order_key(v.w);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) kk[e] = (pos + e < n) ? order_key(src[pos + e]) : 0u;
    }
  };

  uint32_t keys[NC > 0 ? NC : 1][4];
  if constexpr (NC > 0) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if (c < iters) load_keys(c, keys[c]);
      else keys[c][0] = keys[c][1] = keys[c][2] = keys[c][3] = 0u;
    }
  }

  // Radix passes.  prefix/mask describe the candidate set; k_rem counts how
  // many candidates are still to be taken (>= 1).
  uint32_t prefix = 0, mask = 0, k_rem = (uint32_t)K;
  const int shifts[3] = {20, 8, 0};
  const int widths[3] = {12, 12, 8};
  for (int pass = 0; pass < 3; ++pass) {
    const int sh_ = shifts[pass], nb = 1 << widths[pass];
    for (int j = tid; j < nb; j += kThreads) sh.hist[j] = 0;
    __syncthreads();
    auto count = [&](const uint32_t (&kk)[4]) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if ((kk[e] & mask) == prefix && kk[e] != 0u) atomicAdd(&sh.hist[(kk[e] >> sh_) & (nb - 1)], 1u);
    };
    if constexpr (NC > 0) {
#pragma unroll
      for (int c = 0; c < NC; ++c)
        if (c < iters) count(keys[c]);
    } else {
      for (int c = 0; c < iters; ++c) {
        uint32_t kk[4];
        load_keys(c, kk);
        count(kk);
      }
    }
    __syncthreads();
    find_bin(sh, nb, k_rem);
    const uint32_t bin = sh.bin;
    const uint32_t cnt = sh.hist[bin];
    k_rem -= sh.above;
    prefix |= bin << sh_;
    mask |= (uint32_t)(nb - 1) << sh_;
    __syncthreads();
    if (cnt == k_rem) break;                      // the whole bin is taken
  }

  // Ordered emission: chunk c holds positions 4*(c*kThreads + tid) + 0..3,
  // so positions run over (chunk, thread, element).  A group of chunks is
  // scanned at once (one barrier): per chunk a block-wide exclusive scan of
  // the packed (gt, eq) counts, plus running totals over earlier chunks.
  uint32_t gt_run = 0, eq_run = 0;                // counts over earlier chunks
  constexpr int GS = NC >= 16 ? kGroup / 2 : kGroup;   // register budget of the widest variant
  auto emit_group = [&](int c0, int G, const uint32_t (*kk)[4]) {
    uint32_t packed[GS], incl[GS];
#pragma unroll
    for (int g = 0; g < GS; ++g) {
      if (g < G) {
        uint32_t pk = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t m = kk[g][e] & mask;
          const bool valid = kk[g][e] != 0u;
          pk += (valid && m > prefix) ? 1u : 0u;
          pk += (valid && m == prefix) ? 0x10000u : 0u;
        }
        packed[g] = pk;
        incl[g] = wave_incl_scan(pk, lane);
        if (lane == 63) sh.wsum[g * kWaves + wave] = incl[g];
      }
    }
    __syncthreads();
#pragma unroll
    for (int g = 0; g < GS; ++g) {
      if (g < G) {
        uint32_t before = 0, total = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          const uint32_t v = sh.wsum[g * kWaves + w];
          before += (w < wave) ? v : 0u;
          total += v;
        }
        const uint32_t excl = before + incl[g] - packed[g];
        uint32_t g_b = gt_run + (excl & 0xffffu), e_b = eq_run + (excl >> 16);
        const int pos0 = ((c0 + g) * kThreads + tid) * 4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t m = kk[g][e] & mask;
          const bool valid = kk[g][e] != 0u;
          const bool gt = valid && m > prefix, eq = valid && m == prefix;
          if (gt || (eq && e_b < k_rem)) out[g_b + min(e_b, k_rem)] = pos0 + e;
          g_b += gt ? 1u : 0u;
          e_b += eq ? 1u : 0u;
        }
        gt_run += total & 0xffffu;
        eq_run += total >> 16;
      }
    }
    __syncthreads();                              // wsum is reused by the next group
  };
  if constexpr (NC > 0) {
#pragma unroll
    for (int c0 = 0; c0 < NC; c0 += GS)
      if (c0 < iters) emit_group(c0, min(GS, iters - c0), keys + c0);
  } else {
    for (int c0 = 0; c0 < iters; c0 += GS) {
      uint32_t kk[GS][4];
      const int G = min(GS, iters - c0);
#pragma unroll
      for (int g = 0; g < GS; ++g)
        if (g < G) load_keys(c0 + g, kk[g]);
      emit_group(c0, G, kk);
    }
  }
  // K' = min(K, n) = K here (n > K), so no padding is needed.
}

}  // namespace

hipError_t launch_topk(const TopkLaunch& a, hipStream_t s) {
  const int rows = a.B * a.q_count;
  const int n_max = a.Lk - a.Lq + a.q_begin + a.q_count;
  const int chunks = (n_max + 3) / 4;
  const int iters = (chunks + kThreads - 1) / kThreads;
  dim3 grid(rows), block(kThreads);
  if (iters <= 2)
    hipLaunchKernelGGL(topk_kernel<2>, grid, block, 0, s, a);
  else if (iters <= 8)
    hipLaunchKernelGGL(topk_kernel<8>, grid, block, 0, s, a);
  else if (iters <= 16)
    hipLaunchKernelGGL(topk_kernel<16>, grid, block, 0, s, a);
  else
    hipLaunchKernelGGL(topk_kernel<0>, grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace dsa
