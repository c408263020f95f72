// Exact per-row top-k for few long rows, spread over many work-groups.
//
// Same selection as topk.hip (HF model doc "DeepSeek-V3.2", section
// "DeepSeek Sparse Attention (DSA)", item 2: each query keeps its
// index_topk best-scoring positions; larger score first, lower position
// first among equal scores, +0.0 == -0.0; positions emitted ascending).
//
// A decode step has a few dozen rows of tens of thousands of positions; one
// work-group per row would leave most of the 256 CUs idle.  Here each row is
// cut into slices of L = 1024..4096 positions, one work-group per (row,
// slice), and three launches take the place of the passes of a one-group
// radix select (a kernel boundary is the only barrier between the
// work-groups of a row):
//
//  1. tk_hist_kernel: the slice's 12-bit key prefixes (sign, exponent and
//     three mantissa bits of the order-preserving key) into an LDS
//     histogram, whose non-empty bins are added into the row's histogram in
//     global memory (zeroed by the indexer kernel that wrote the scores).
//  2. tk_classify_kernel: every work-group reads the row histogram and
//     finds the bin b1 holding the K-th largest key and how many keys r1 the
//     selection still needs from it; it then keeps the slice's keys with
//     prefix >= b1 (all of them chosen except those in b1), in position
//     order with their positions, and records how many are above b1 and in
//     b1.
//  3. tk_emit_kernel: every work-group finishes the threshold from the
//     row's kept keys in b1 alone (a few hundred for index scores): two
//     10-bit radix passes give the exact threshold key T and how many keys
//     equal to T are taken (the lowest positions first); per-slice counts
//     then give each slice's first output slot, and the work-group writes
//     its slice's chosen positions, in order, from its kept list.
//
// Exact: fewer than K keys lie in bins above b1 and each of them beats every
// key in or below b1, so all of them are chosen and none below b1 is; the
// rest is the ordinary ordered selection among the keys of b1.
#include <atomic>

#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kT = 256;              // threads per work-group
constexpr int kW = kT / 64;          // waves
constexpr int kBins1 = 4096;         // first level: key bits 31..20
constexpr int kBins2 = 1024;         // then bits 19..10 and 9..0
constexpr int kMaxSl = kMaxTopkSlices;
constexpr int kHead = kTopkRowHeadWords;   // per row: histogram, then barrier counters

// Order-preserving key (-0.0 as +0.0).  Positions beyond the row hold no
// element; they are marked with key 0, which no finite score or infinity
// maps to.
__device__ __forceinline__ uint32_t skey(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive block-wide scan of one value per thread; *total gets the sum.
// ws holds kW words of scratch.  All threads must call; contains barriers.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* ws, uint32_t* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t incl = wave_incl_scan(v);
  if (lane == 63) ws[wave] = incl;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kW; ++w) {
    const uint32_t x = ws[w];
    before += w < wave ? x : 0u;
    tot += x;
  }
  __syncthreads();                               // ws may be reused right after
  *total = tot;
  return before + incl - v;
}

// Row and slice of this work-group.  Work-groups are dealt to the 8 XCDs
// round-robin by linear id; when the row count allows it, all slices of a
// row go to one XCD so the three launches meet the row's data in one L2.
struct RowSlice {
  int r, s;
};
__device__ __forceinline__ RowSlice row_slice(int P, int rows) {
  const int lin = blockIdx.x;
  RowSlice rs;
  if ((rows & 7) == 0) {
    const int loc = lin >> 3;
    rs.r = (lin & 7) + 8 * (loc / P);
    rs.s = loc - (loc / P) * P;
  } else {
    rs.r = lin / P;
    rs.s = lin - rs.r * P;
  }
  return rs;
}

// Keys of this thread's part of slice s: positions p0 + 4*CPT*tid + 4c + e
// (CPT consecutive 4-position chunks per thread, so a thread's keys are in
// position order and threads follow each other).  Beyond n: key 0.
template <int CPT, bool VEC>
__device__ __forceinline__ void load_slice(const float* row, int p0, int n, uint32_t (&k)[CPT][4]) {
  const int base = p0 + 4 * CPT * (int)threadIdx.x;
  if constexpr (VEC) {
    f32x4 v[CPT];
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int p = base + 4 * c;
      if (p + 3 < n) {
        v[c] = *reinterpret_cast<const f32x4*>(row + p);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[c][e] = p + e < n ? row[p + e] : 0.f;
      }
    }
#pragma unroll
    for (int c = 0; c < CPT; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) k[c][e] = base + 4 * c + e < n ? skey(v[c][e]) : 0u;
  } else {
#pragma unroll
    for (int c = 0; c < CPT; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int p = base + 4 * c + e;
        k[c][e] = p < n ? skey(row[p]) : 0u;
      }
  }
}

struct RowInfo {
  int b, i, n;
};
__device__ __forceinline__ RowInfo row_info(const TopkLaunch& a, int r) {
  RowInfo ri;
  ri.b = r / a.q_count;
  ri.i = a.q_begin + (r - ri.b * a.q_count);
  ri.n = a.Lk - a.Lq + ri.i + 1;
  return ri;
}

// ---------------------------------------------------------------- 1 ------
template <int CPT, bool VEC>
__global__ __launch_bounds__(kT) void tk_hist_kernel(TopkLaunch a) {
  __shared__ uint32_t h[kBins1];
  const int rows = a.B * a.q_count;
  const RowSlice rs = row_slice(a.sl_count, rows);
  const RowInfo ri = row_info(a, rs.r);
  const int p0 = rs.s * (CPT * 4 * kT);
  if (ri.n <= a.K || p0 >= ri.n) return;         // whole row chosen / empty slice
  const int tid = threadIdx.x;
  uint32_t k[CPT][4];
  load_slice<CPT, VEC>(a.scores + (int64_t)rs.r * a.row_stride, p0, ri.n, k);
#pragma unroll
  for (int j = 0; j < kBins1 / (4 * kT); ++j) st16(&h[4 * (tid + kT * j)], u32x4{0u, 0u, 0u, 0u});
  __syncthreads();
#pragma unroll
  for (int c = 0; c < CPT; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (k[c][e]) atomicAdd(&h[k[c][e] >> 20], 1u);
  __syncthreads();
  uint32_t* gh = a.sl_hist + (int64_t)rs.r * kHead;
#pragma unroll
  for (int j = 0; j < kBins1 / kT; ++j) {
    const uint32_t v = h[tid + kT * j];
    if (v) atomicAdd(&gh[tid + kT * j], v);
  }
}

// Bin holding the k-th largest element (1 <= k <= total) of a histogram of
// nb = PER * kT bins, thread t owning bins nb-1-PER*t down to nb-PER*(t+1):
// returns the bin and, in *above, the number of elements in higher bins.
// cnt[] holds this thread's counts, highest bin first.  Contains barriers.
// LDS histograms that find_bin reads as runs of PER consecutive bins per
// thread: a pad word after every run puts neighbouring lanes' runs in
// different banks (unpadded, lanes 16 or 4 words apart share a few banks).
template <int PER>
__device__ __forceinline__ int padded(int bin) { return bin + bin / PER; }
constexpr int kPad1 = kBins1 + kBins1 / 16;     // 4096 bins read 16 per thread
constexpr int kPad2 = kBins2 + kBins2 / 4;      // 1024 bins read 4 per thread

template <int PER>
__device__ __forceinline__ uint32_t find_bin(const uint32_t (&cnt)[PER], uint32_t k, uint32_t* ws, uint32_t* res,
                                             uint32_t* above) {
  const int tid = threadIdx.x;
  if (tid == 0) {                                // defined even if k exceeded the total
    res[0] = 0u;
    res[1] = 0u;
  }
  uint32_t local = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) local += cnt[j];
  uint32_t tot;
  const uint32_t before = block_excl_scan(local, ws, &tot);
  if (before < k && k <= before + local) {
    uint32_t acc = before;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      if (acc < k && k <= acc + cnt[j]) {
        res[0] = (uint32_t)(PER * kT - 1 - PER * tid - j);
        res[1] = acc;
      }
      acc += cnt[j];
    }
  }
  __syncthreads();
  *above = res[1];
  const uint32_t bin = res[0];
  __syncthreads();                               // res may be reused right after
  return bin;
}

// ---------------------------------------------------------------- 2 ------
template <int CPT, bool VEC>
__global__ __launch_bounds__(kT) void tk_classify_kernel(TopkLaunch a) {
  __shared__ uint32_t ws[kW];
  __shared__ uint32_t res[2];
  const int rows = a.B * a.q_count;
  const RowSlice rs = row_slice(a.sl_count, rows);
  const RowInfo ri = row_info(a, rs.r);
  const int L = CPT * 4 * kT;
  const int p0 = rs.s * L;
  if (ri.n <= a.K || p0 >= ri.n) return;
  const int tid = threadIdx.x;
  uint32_t k[CPT][4];
  load_slice<CPT, VEC>(a.scores + (int64_t)rs.r * a.row_stride, p0, ri.n, k);
  // the row histogram, highest bins first: thread t owns 16 bins
  const uint32_t* gh = a.sl_hist + (int64_t)rs.r * kHead;
  uint32_t cnt[16];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const u32x4 v = ld16(&gh[kBins1 - 16 * (tid + 1) + 12 - 4 * q]);
    cnt[4 * q] = v.w;
    cnt[4 * q + 1] = v.z;
    cnt[4 * q + 2] = v.y;
    cnt[4 * q + 3] = v.x;
  }
  uint32_t above;
  const uint32_t b1 = find_bin<16>(cnt, (uint32_t)a.K, ws, res, &above);
  // keep keys with prefix >= b1, in position order
  uint32_t ngt = 0, neq = 0;
#pragma unroll
  for (int c = 0; c < CPT; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t d = k[c][e] >> 20;
      ngt += (k[c][e] != 0u && d > b1) ? 1u : 0u;
      neq += (k[c][e] != 0u && d == b1) ? 1u : 0u;
    }
  uint32_t tot;
  const uint32_t excl = block_excl_scan(ngt | (neq << 16), ws, &tot);
  uint32_t o = (excl & 0xffffu) + (excl >> 16), oc = excl >> 16;
  const int64_t slot = (int64_t)rs.r * a.sl_count + rs.s;
  uint32_t* list = a.sl_list + slot * (2 * L);
  uint32_t* cand = a.sl_cand + slot * L;
  const int pbase = p0 + 4 * CPT * tid;
#pragma unroll
  for (int c = 0; c < CPT; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (k[c][e] != 0u && (k[c][e] >> 20) >= b1) {
        *reinterpret_cast<u32x2*>(&list[2 * o]) = u32x2{k[c][e], (uint32_t)(pbase + 4 * c + e)};
        ++o;
        if ((k[c][e] >> 20) == b1) cand[oc++] = k[c][e];
      }
  if (tid == 0) {
    int32_t* info = a.sl_info + ((int64_t)rs.r * kMaxSl + rs.s) * 2;
    info[0] = (int32_t)(tot & 0xffffu);
    info[1] = (int32_t)(tot >> 16);
    if (rs.s == 0) {
      int32_t* rinfo = a.sl_rowinfo + (int64_t)rs.r * 4;
      rinfo[0] = (int32_t)b1;
      rinfo[1] = a.K - (int32_t)above;
    }
  }
}

// ---------------------------------------------------------------- 3 ------
constexpr int kCandRegs = 16;        // candidates held per thread (4096 per work-group)

struct EmitShared {
  uint32_t h[kPad2];               // the 1024-bin passes (padded runs of 4)
  uint32_t cstart[kMaxSl + 1];     // flattened start of each slice's candidates
  uint32_t gt[kMaxSl];             // candidates above T per slice
  uint32_t eq[kMaxSl];             // candidates equal to T per slice
  uint32_t ws[kW];
  uint32_t res[2];
};

// Slice holding flattened candidate c (cstart[] ascending, cstart[0] = 0).
__device__ __forceinline__ int slice_of(const uint32_t* start, int np, uint32_t c) {
  int lo = 0, hi = np;                           // start[lo] <= c < start[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (start[mid] <= c) lo = mid;
    else hi = mid;
  }
  return lo;
}

__global__ __launch_bounds__(kT) void tk_emit_kernel(TopkLaunch a, int L) {
  __shared__ EmitShared sh;
  const int rows = a.B * a.q_count;
  const int P = a.sl_count;
  const RowSlice rs = row_slice(P, rows);
  const RowInfo ri = row_info(a, rs.r);
  const int tid = threadIdx.x;
  const int K = a.K;
  int32_t* out = a.out + ((int64_t)ri.b * a.Lq + ri.i) * K;
  if (ri.n <= K) {                               // every visible position, then -1
    for (int j = rs.s * kT + tid; j < K; j += P * kT) out[j] = j < ri.n ? j : -1;
    return;
  }
  const int np = (ri.n + L - 1) / L;             // slices holding elements
  if (rs.s >= np) return;
  const int32_t* info = a.sl_info + (int64_t)rs.r * kMaxSl * 2;
  const int64_t row_slot = (int64_t)rs.r * P;
  // Everything this work-group reads is issued at once: the per-slice
  // counts, the row's threshold bin, this slice's kept list (the whole
  // L-entry buffer, masked by its count later) and a fixed share of every
  // slice's candidate buffer (thread t: slice t % np, entries t / np,
  // + tps, ...), so the work-group waits for memory once.
  const uint32_t* list = a.sl_list + (row_slot + rs.s) * (2 * L);
  const uint32_t* cand_row = a.sl_cand + row_slot * L;
  const int32_t* rinfo = a.sl_rowinfo + (int64_t)rs.r * 4;
  u32x2 kept[kCandRegs];
#pragma unroll
  for (int u = 0; u < kCandRegs; ++u)
    kept[u] = u * kT < L ? *reinterpret_cast<const u32x2*>(&list[2 * (u * kT + tid)]) : u32x2{0u, 0u};
  const int tps = np <= kT ? kT / np : 0;        // threads per slice for the candidates
  const int my_sl = tps ? tid % np : 0;
  const int my_j0 = tps ? tid / np : 0;
  const bool my_on = tps && tid < np * tps;
  uint32_t ck[kCandRegs];
  uint16_t csl[kCandRegs];
#pragma unroll
  for (int u = 0; u < kCandRegs; ++u) {
    const int jj = my_j0 + u * tps;
    ck[u] = my_on && jj < L ? cand_row[(int64_t)my_sl * L + jj] : 0u;
    csl[u] = (uint16_t)my_sl;
  }
  const uint32_t my_ce = my_on ? (uint32_t)info[2 * my_sl + 1] : 0u;
  const uint32_t ms = (uint32_t)(info[2 * rs.s] + info[2 * rs.s + 1]);
  uint32_t ce[2], g0[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int sl = 2 * tid + u;
    ce[u] = sl < np ? (uint32_t)info[2 * sl + 1] : 0u;
    g0[u] = sl < np ? (uint32_t)info[2 * sl] : 0u;
  }
  const uint32_t b1 = (uint32_t)rinfo[0];
  const uint32_t r1 = (uint32_t)rinfo[1];
#pragma unroll
  for (int u = 0; u < kCandRegs; ++u)
    if ((uint32_t)(my_j0 + u * tps) >= my_ce) ck[u] = 0u;        // 0: no candidate
  // did every slice's candidates fit the fixed shares?  (index scores: a
  // few dozen per slice; a row of many equal scores may not)
  const bool spill = !tps || ce[0] > (uint32_t)(tps * kCandRegs) || ce[1] > (uint32_t)(tps * kCandRegs);
  const bool held = !__syncthreads_or(spill);
  uint32_t C = 0;
  if (!held) {                                   // flattened starts for the batched re-reads
    const uint32_t cs0 = block_excl_scan(ce[0] + ce[1], sh.ws, &C);
    if (2 * tid < np) sh.cstart[2 * tid] = cs0;
    if (2 * tid + 1 < np) sh.cstart[2 * tid + 1] = cs0 + ce[0];
    if (tid == 0) sh.cstart[np] = C;
    __syncthreads();
  }
  auto load_batch = [&](uint32_t c0) {
#pragma unroll
    for (int u = 0; u < kCandRegs; ++u) {
      const uint32_t c = c0 + (uint32_t)(u * kT + tid);
      int sl = 0;
      uint32_t key = 0u;                          // 0: no candidate
      if (c < C) {
        sl = slice_of(sh.cstart, np, c);
        key = cand_row[(int64_t)sl * L + (c - sh.cstart[sl])];
      }
      ck[u] = key;
      csl[u] = (uint16_t)sl;
    }
  };
  auto for_each = [&](auto&& f) {
    if (held) {
#pragma unroll
      for (int u = 0; u < kCandRegs; ++u)
        if (ck[u]) f(ck[u], (int)csl[u]);
    } else {
      for (uint32_t c0 = 0; c0 < C; c0 += kCandRegs * kT) {
        load_batch(c0);
#pragma unroll
        for (int u = 0; u < kCandRegs; ++u)
          if (ck[u]) f(ck[u], (int)csl[u]);
      }
    }
  };
  // two 10-bit passes over the candidates
  uint32_t prefix = b1, need = r1;
#pragma unroll 1
  for (int pass = 0; pass < 2; ++pass) {
    const int shift = pass == 0 ? 10 : 0;
    const int pshift = pass == 0 ? 20 : 10;
#pragma unroll
    for (int b = tid; b < kPad2; b += kT) sh.h[b] = 0u;
    __syncthreads();
    for_each([&](uint32_t key, int) {
      if ((key >> pshift) == prefix) atomicAdd(&sh.h[padded<4>((key >> shift) & (kBins2 - 1))], 1u);
    });
    __syncthreads();
    uint32_t cnt[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) cnt[j] = sh.h[padded<4>(kBins2 - 1 - 4 * tid - j)];
    uint32_t above;
    const uint32_t bin = find_bin<4>(cnt, need, sh.ws, sh.res, &above);
    prefix = (prefix << 10) | bin;
    need -= above;
  }
  const uint32_t T = prefix;                     // the K-th largest key
  const uint32_t r_eq = need;                    // keys equal to T that are taken
  // per slice: candidates above T and equal to T
  for (int sl = tid; sl < np; sl += kT) {
    sh.gt[sl] = 0u;
    sh.eq[sl] = 0u;
  }
  __syncthreads();
  for_each([&](uint32_t key, int sl) {
    if (key > T) atomicAdd(&sh.gt[sl], 1u);
    else if (key == T) atomicAdd(&sh.eq[sl], 1u);
  });
  __syncthreads();
  // equal keys go to the lowest positions first: slice s takes
  // clamp(r_eq - (equal keys of earlier slices), 0, eq[s])
  uint32_t eqv[2], gtv[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int sl = 2 * tid + u;
    eqv[u] = sl < np ? sh.eq[sl] : 0u;
    gtv[u] = sl < np ? g0[u] + sh.gt[sl] : 0u;
  }
  uint32_t tmp;
  const uint32_t eq_before0 = block_excl_scan(eqv[0] + eqv[1], sh.ws, &tmp);
  uint32_t take[2], sel[2];
  {
    uint32_t eb = eq_before0;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      take[u] = eb >= r_eq ? 0u : min(r_eq - eb, eqv[u]);
      sel[u] = gtv[u] + take[u];
      eb += eqv[u];
    }
  }
  const uint32_t off0 = block_excl_scan(sel[0] + sel[1], sh.ws, &tmp);
  // this slice's first output slot and equal-key quota
  if (2 * tid == rs.s || 2 * tid + 1 == rs.s) {
    const int u = rs.s - 2 * tid;
    sh.res[0] = off0 + (u ? sel[0] : 0u);
    sh.res[1] = take[u];
  }
  __syncthreads();
  const uint32_t off = sh.res[0], quota = sh.res[1];
  // ordered emission from the slice's kept list (round u: entries u*kT + tid)
  uint32_t gt_run = 0, eq_run = 0;
#pragma unroll
  for (int u = 0; u < kCandRegs; ++u) {
    if ((uint32_t)(u * kT) >= ms) break;         // uniform
    const uint32_t j = (uint32_t)(u * kT + tid);
    const uint32_t key = kept[u].x, pos = kept[u].y;
    const bool gt = j < ms && key > T, eq = j < ms && key == T;
    uint32_t tot;
    const uint32_t excl = block_excl_scan((gt ? 1u : 0u) | (eq ? 0x10000u : 0u), sh.ws, &tot);
    const uint32_t g_b = gt_run + (excl & 0xffffu), e_b = eq_run + (excl >> 16);
    const uint32_t slot = off + g_b + min(e_b, quota);
    if ((gt || (eq && e_b < quota)) && slot < (uint32_t)K) out[slot] = (int32_t)pos;
    gt_run += tot & 0xffffu;
    eq_run += tot >> 16;
  }
}

// ------------------------------------------------------- one launch ------
// The same selection in one launch when every work-group of the grid is
// resident at once (the host checks occupancy x CUs against the grid): the
// work-groups of a row meet at two row barriers instead of kernel
// boundaries, and each keeps its slice's keys in registers from the first
// load to its emission.
//  - histogram: as tk_hist_kernel; barrier 1.
//  - threshold bin b1 from the row histogram; the slice's keys in b1 go to
//    its candidate buffer and its counts (above b1, in b1) to the row's
//    table; barrier 2.
//  - every work-group reads every slice's candidates and counts, finds T
//    and the per-slice offsets and equal-key quotas (as tk_emit_kernel), and
//    writes its own chosen positions from registers.
// A barrier is an arrival counter in the row head (zero on entry) and a
// bounded wait: a work-group gives up after 2^18 polls (a fraction of a
// second), so a grid that was not resident after all ends with undefined
// indices for that row instead of hanging.
// Everything the work-groups of a row exchange goes through device-scope
// atomics: histogram adds, and relaxed atomic stores and loads (which the
// compiler issues with the system-coherent cache bit, so they complete at
// and read from the device's coherence point rather than a per-XCD L2).
// Each wave waits for its own stores and atomics to complete (a work-group
// barrier alone does not) before the work-group barrier that precedes the
// arrival, and readers load only after seeing every arrival, so no L2
// write-back or invalidation is needed.
constexpr int kSpinMax = 1 << 18;

__device__ __forceinline__ void row_barrier(uint32_t* ctr, uint32_t target) {
  wait_vmcnt<0>();                               // this wave's stores and atomics have completed
  __syncthreads();                               // ... and every other wave's
  if (threadIdx.x == 0) {
    __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int spin = 0; spin < kSpinMax; ++spin) {
      if (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= target) break;
      __builtin_amdgcn_s_sleep(1);
    }
  }
  __syncthreads();
}
__device__ __forceinline__ uint32_t coh_load(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void coh_store(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// 16-byte loads that bypass the non-coherent cache levels (sc1), as the
// agent-scope atomic loads do, for data other work-groups of the launch
// wrote; a buffer resource keeps reads past `bytes` at zero.
constexpr int kSc1 = 16;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t coh_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

struct CoopShared {
  uint32_t h[kPad1];       // the slice's histogram, then the row's (padded), then the 1024-bin passes
  uint32_t gt[kMaxSl];
  uint32_t eq[kMaxSl];
  uint32_t ws[kW];
  uint32_t res[2];
};

template <int CPT, bool VEC>
__global__ __launch_bounds__(kT) void tk_coop_kernel(TopkLaunch a) {
  __shared__ CoopShared sh;
  const int rows = a.B * a.q_count;
  const int P = a.sl_count;
  constexpr int L = CPT * 4 * kT;
  const RowSlice rs = row_slice(P, rows);
  const RowInfo ri = row_info(a, rs.r);
  const int tid = threadIdx.x;
  const int K = a.K;
  int32_t* out = a.out + ((int64_t)ri.b * a.Lq + ri.i) * K;
  if (ri.n <= K) {                               // every visible position, then -1
    for (int j = rs.s * kT + tid; j < K; j += P * kT) out[j] = j < ri.n ? j : -1;
    return;
  }
  const int np = (ri.n + L - 1) / L;             // work-groups of this row that hold elements
  if (rs.s >= np) return;
  const int p0 = rs.s * L;
  uint32_t k[CPT][4];
  load_slice<CPT, VEC>(a.scores + (int64_t)rs.r * a.row_stride, p0, ri.n, k);
  uint32_t* head = a.sl_hist + (int64_t)rs.r * kHead;
  // 1. histogram of 12-bit prefixes, merged into the row head
#pragma unroll
  for (int j = 0; j < kBins1 / (4 * kT); ++j) st16(&sh.h[4 * (tid + kT * j)], u32x4{0u, 0u, 0u, 0u});
  __syncthreads();
#pragma unroll
  for (int c = 0; c < CPT; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (k[c][e]) atomicAdd(&sh.h[k[c][e] >> 20], 1u);
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kBins1 / kT; ++j) {
    const uint32_t v = sh.h[tid + kT * j];
    if (v) atomicAdd(&head[tid + kT * j], v);
  }
  row_barrier(head + kBins1, (uint32_t)np);
  // 2. threshold bin (the row histogram comes in through LDS: coalesced
  // 16-byte loads, then 16 consecutive bins per thread); this slice's
  // candidates (keys in b1) and counts
  {
    const __amdgpu_buffer_rsrc_t hr = coh_rsrc(head, kBins1 * 4);
#pragma unroll
    for (int j = 0; j < kBins1 / (4 * kT); ++j) {
      const int c = tid + kT * j;
      const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(hr, 16 * c, 0, kSc1);
#pragma unroll
      for (int e = 0; e < 4; ++e) sh.h[padded<16>(4 * c) + e] = v[e];   // bins 4c..4c+3 share a run
    }
  }
  __syncthreads();
  uint32_t cnt[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) cnt[j] = sh.h[padded<16>(kBins1 - 1 - 16 * tid - j)];
  uint32_t above;
  const uint32_t b1 = find_bin<16>(cnt, (uint32_t)K, sh.ws, sh.res, &above);
  const uint32_t r1 = (uint32_t)K - above;
  uint32_t ngt = 0, neq = 0;
#pragma unroll
  for (int c = 0; c < CPT; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t d = k[c][e] >> 20;
      ngt += (k[c][e] != 0u && d > b1) ? 1u : 0u;
      neq += (k[c][e] != 0u && d == b1) ? 1u : 0u;
    }
  uint32_t tot;
  const uint32_t excl = block_excl_scan(ngt | (neq << 16), sh.ws, &tot);
  const int64_t row_slot = (int64_t)rs.r * P;
  uint32_t* cand_row = a.sl_cand + row_slot * L;
  {
    uint32_t oc = excl >> 16;
    uint32_t* cand = cand_row + (int64_t)rs.s * L;
#pragma unroll
    for (int c = 0; c < CPT; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (k[c][e] != 0u && (k[c][e] >> 20) == b1) coh_store(&cand[oc++], k[c][e]);
  }
  uint32_t* info = reinterpret_cast<uint32_t*>(a.sl_info) + (int64_t)rs.r * kMaxSl * 2;
  if (tid == 0) {
    coh_store(&info[2 * rs.s], tot & 0xffffu);
    coh_store(&info[2 * rs.s + 1], tot >> 16);
  }
  row_barrier(head + kBins1 + 1, (uint32_t)np);
  // 3. every slice's counts and candidates: tps threads per slice, thread j
  // of a slice holding its candidates 4(j + tps u) .. +3 (16-byte loads,
  // a slice's threads reading consecutive bytes)
  const int tps = np <= kT ? kT / np : 0;
  const int my_sl = tps ? tid / tps : 0;
  const int my_j = tps ? tid - my_sl * tps : 0;
  const bool my_on = tps && tid < np * tps;
  uint32_t ck[kCandRegs];
  static_assert(kCandRegs % 4 == 0, "candidates load in groups of four");
  {
    const __amdgpu_buffer_rsrc_t cr = coh_rsrc(cand_row, (uint32_t)np * (uint32_t)L * 4u);
#pragma unroll
    for (int u = 0; u < kCandRegs / 4; ++u) {
      const int jj = 4 * (my_j + u * tps);
      const u32x4 v = my_on && jj < L ? __builtin_amdgcn_raw_buffer_load_b128(cr, 4 * (my_sl * L + jj), 0, kSc1)
                                      : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < 4; ++e) ck[4 * u + e] = v[e];
    }
  }
  const uint32_t my_ce = my_on ? coh_load(&info[2 * my_sl + 1]) : 0u;
  uint32_t ce[2], g0[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int sl = 2 * tid + u;
    ce[u] = sl < np ? coh_load(&info[2 * sl + 1]) : 0u;
    g0[u] = sl < np ? coh_load(&info[2 * sl]) : 0u;
  }
#pragma unroll
  for (int u = 0; u < kCandRegs; ++u)
    if ((uint32_t)(4 * (my_j + (u / 4) * tps) + (u % 4)) >= my_ce) ck[u] = 0u;
  const bool spill = !tps || ce[0] > (uint32_t)(tps * kCandRegs) || ce[1] > (uint32_t)(tps * kCandRegs);
  const bool held = !__syncthreads_or(spill);
  // candidates that did not fit the fixed shares: every slice's buffer is
  // walked in batches of kT entries per slice on each pass
  auto for_each = [&](auto&& f) {
    if (held) {
#pragma unroll
      for (int u = 0; u < kCandRegs; ++u)
        if (ck[u]) f(ck[u], my_sl);
    } else {
      for (int sl = 0; sl < np; ++sl) {
        const uint32_t n_sl = coh_load(&info[2 * sl + 1]);
        for (uint32_t j = tid; j < n_sl; j += kT) f(coh_load(&cand_row[(int64_t)sl * L + j]), sl);
      }
    }
  };
  uint32_t prefix = b1, need = r1;
#pragma unroll 1
  for (int pass = 0; pass < 2; ++pass) {
    const int shift = pass == 0 ? 10 : 0;
    const int pshift = pass == 0 ? 20 : 10;
#pragma unroll
    for (int b = tid; b < kPad2; b += kT) sh.h[b] = 0u;
    __syncthreads();
    for_each([&](uint32_t key, int) {
      if ((key >> pshift) == prefix) atomicAdd(&sh.h[padded<4>((key >> shift) & (kBins2 - 1))], 1u);
    });
    __syncthreads();
    uint32_t c4[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) c4[j] = sh.h[padded<4>(kBins2 - 1 - 4 * tid - j)];
    uint32_t ab;
    const uint32_t bin = find_bin<4>(c4, need, sh.ws, sh.res, &ab);
    prefix = (prefix << 10) | bin;
    need -= ab;
  }
  const uint32_t T = prefix, r_eq = need;
  for (int sl = tid; sl < np; sl += kT) {
    sh.gt[sl] = 0u;
    sh.eq[sl] = 0u;
  }
  __syncthreads();
  for_each([&](uint32_t key, int sl) {
    if (key > T) atomicAdd(&sh.gt[sl], 1u);
    else if (key == T) atomicAdd(&sh.eq[sl], 1u);
  });
  __syncthreads();
  uint32_t eqv[2], gtv[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int sl = 2 * tid + u;
    eqv[u] = sl < np ? sh.eq[sl] : 0u;
    gtv[u] = sl < np ? g0[u] + sh.gt[sl] : 0u;
  }
  uint32_t tmp;
  const uint32_t eq_before0 = block_excl_scan(eqv[0] + eqv[1], sh.ws, &tmp);
  uint32_t take[2], sel[2];
  {
    uint32_t eb = eq_before0;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      take[u] = eb >= r_eq ? 0u : min(r_eq - eb, eqv[u]);
      sel[u] = gtv[u] + take[u];
      eb += eqv[u];
    }
  }
  const uint32_t off0 = block_excl_scan(sel[0] + sel[1], sh.ws, &tmp);
  if (2 * tid == rs.s || 2 * tid + 1 == rs.s) {
    const int u = rs.s - 2 * tid;
    sh.res[0] = off0 + (u ? sel[0] : 0u);
    sh.res[1] = take[u];
  }
  __syncthreads();
  const uint32_t off = sh.res[0], quota = sh.res[1];
  // emission from registers: this thread's keys are positions
  // p0 + 4*CPT*tid + 4c + e, in position order across threads
  uint32_t g_n = 0, e_n = 0;
#pragma unroll
  for (int c = 0; c < CPT; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      g_n += (k[c][e] != 0u && k[c][e] > T) ? 1u : 0u;
      e_n += (k[c][e] != 0u && k[c][e] == T) ? 1u : 0u;
    }
  const uint32_t ex = block_excl_scan(g_n | (e_n << 16), sh.ws, &tmp);
  uint32_t g_b = ex & 0xffffu, e_b = ex >> 16;
  const int pbase = p0 + 4 * CPT * tid;
#pragma unroll
  for (int c = 0; c < CPT; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t key = k[c][e];
      const bool gt = key != 0u && key > T, eq = key != 0u && key == T;
      const uint32_t slot = off + g_b + min(e_b, quota);
      if ((gt || (eq && e_b < quota)) && slot < (uint32_t)K) out[slot] = pbase + 4 * c + e;
      g_b += gt ? 1u : 0u;
      e_b += eq ? 1u : 0u;
    }
}

__global__ __launch_bounds__(kT) void tk_zero_kernel(uint32_t* p, int64_t n4) {
  const int64_t j = (int64_t)blockIdx.x * kT + threadIdx.x;
  if (j < n4) st16(p + 4 * j, u32x4{0u, 0u, 0u, 0u});
}

template <int CPT, bool VEC>
void launch_sliced_t(const TopkLaunch& a, hipStream_t s) {
  const int grid = a.B * a.q_count * a.sl_count;
  launch_kernel(tk_hist_kernel<CPT, VEC>, dim3(grid), dim3(kT), 0, s, a);
  launch_kernel(tk_classify_kernel<CPT, VEC>, dim3(grid), dim3(kT), 0, s, a);
  launch_kernel(tk_emit_kernel, dim3(grid), dim3(kT), 0, s, a, CPT * 4 * kT);
}

template <int CPT, bool VEC>
void launch_coop_t(const TopkLaunch& a, hipStream_t s) {
  const int grid = a.B * a.q_count * a.sl_count;
  launch_kernel(tk_coop_kernel<CPT, VEC>, dim3(grid), dim3(kT), 0, s, a);
}

// Work-groups of tk_coop_kernel<CPT, VEC> the current device holds at once
// (occupancy per CU x CUs), computed once per device and slice length.
template <int CPT, bool VEC>
int64_t coop_capacity() {
  constexpr int kMaxDev = 64;
  static std::atomic<int64_t> cap[kMaxDev];      // 0: not yet computed
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return 0;
  int64_t c = cap[dev].load(std::memory_order_relaxed);
  if (c == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, tk_coop_kernel<CPT, VEC>, kT, 0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    c = (int64_t)per_cu * cus;
    cap[dev].store(c > 0 ? c : -1, std::memory_order_relaxed);
  }
  return c;
}

template <int CPT, bool VEC>
void launch_len(const TopkLaunch& a, hipStream_t s) {
  const int64_t grid = (int64_t)a.B * a.q_count * a.sl_count;
  if (grid <= coop_capacity<CPT, VEC>()) launch_coop_t<CPT, VEC>(a, s);
  else launch_sliced_t<CPT, VEC>(a, s);
}

template <bool VEC>
hipError_t launch_sliced_v(const TopkLaunch& a, hipStream_t s) {
  switch (a.sl_len) {
    case 1024: launch_len<1, VEC>(a, s); break;
    case 2048: launch_len<2, VEC>(a, s); break;
    case 4096: launch_len<4, VEC>(a, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipSuccess;
}

}  // namespace

int topk_sliced_len(int rows, int n_max, int K) {
  // One work-group per row is enough once rows fill the CUs.  Below 65536
  // positions a row is cheaper in one work-group than in slices that meet
  // at barriers: each cross-CU round trip costs microseconds (32768
  // positions, 32 rows: 13.4 us in one work-group per row, 16.2 us sliced
  // in one launch, 18.4 us in three; 131072 positions, 8 rows: 18.1 us
  // sliced against 23 us for the earlier two-stage form).
  if (rows > 128 || n_max <= K || n_max < 65536) return 0;
  int L = 4096;
  while (L > 1024 && (int64_t)rows * ((n_max + L - 1) / L) < 256) L /= 2;
  if ((n_max + L - 1) / L > kMaxSl) return 0;
  return L;
}

size_t topk_sliced_bytes(int rows, int n_max, int L, size_t* hist_bytes) {
  const int P = (n_max + L - 1) / L;
  *hist_bytes = (size_t)rows * kHead * 4;
  // hist, per-slice counts, per-row threshold bin, kept lists (key,
  // position), candidate keys
  return *hist_bytes + (size_t)rows * kMaxSl * 2 * 4 + (size_t)rows * 4 * 4 + (size_t)rows * P * L * 12;
}

hipError_t launch_topk_sliced(const TopkLaunch& a, bool zero_hist, hipStream_t s) {
  if (a.sl_count < 1 || a.sl_count > kMaxSl || !a.sl_hist || !a.sl_info || !a.sl_rowinfo || !a.sl_list ||
      !a.sl_cand)
    return hipErrorInvalidValue;
  if (zero_hist) {
    const int64_t n4 = (int64_t)a.B * a.q_count * kHead / 4;
    launch_kernel(tk_zero_kernel, dim3((unsigned)((n4 + kT - 1) / kT)), dim3(kT), 0, s, a.sl_hist, n4);
  }
  const hipError_t e = a.vec_ok ? launch_sliced_v<true>(a, s) : launch_sliced_v<false>(a, s);
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

}  // namespace dsa
