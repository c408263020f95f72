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
// Index scores crowd into a few exponents, so many lanes of one atomic
// instruction hit the same bin; the first pass's histogram therefore keeps
// C copies (lane l adds to copy l % C), laid out copy-major with a stride of
// 4096 + 4 words so the copies of one bin sit in different banks and a
// thread's run of 4 bins is one aligned 16-byte read.  Later passes count
// one bin's elements into a single copy.
// The selection is {key > T} plus the first r positions with key == T; when
// the last pass takes its bin whole it is simply {key >= prefix}.
// Rows held in registers (4 consecutive positions per 16-byte load) write
// two bitmaps over positions, "above T" and "equal to T", one 32-position
// word per 8 lanes (DPP OR of their 4-bit groups); one thread per word then
// turns a block-wide scan of the word counts into output slots, keeping the
// equal positions while fewer than r came before, and writes the positions
// of its set bits.  Longer rows, re-read from memory each pass, use an
// ordered pass over the elements instead: for a chosen element at position
// x its slot is  #(key > T before x) + min(#(key == T before x), r), from
// block-wide scans of packed counts (one barrier per group of 8 chunks).
// Slots go to LDS first and leave in one coalesced copy (K <= 4096).
#include <type_traits>

#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kBins = 4096;
constexpr int kGroup = 8;            // chunks per emission group

template <int NC, int C>
struct Shared {
  static constexpr int kStride = kBins + 4;   // bin j, copy c at c * kStride + j
  static constexpr int kWords = NC > 0 ? NC * kThreads * 4 / 32 : 1;   // bitmap words
  // pass 1: C copies; then copy 0 holds pass 2; at the end the output stage
  alignas(16) uint32_t hist[C * kStride];
  alignas(16) uint32_t h3[256];     // pass 3
  uint32_t gt_bits[kWords];         // position x: bit x % 32 of word x / 32
  uint32_t eq_bits[kWords];
  alignas(16) uint32_t wsum[kGroup * kWaves];
  uint32_t bin;                     // chosen bin of the current pass
  uint32_t above;                   // elements in bins above it
  uint32_t cnt;                     // elements in it
};

// Sum of the per-wave totals ws[0..kWaves) over the waves before `wave`:
// lane l of each 16-lane row reads total l (or 0), a row scan leaves the sum
// in lane 15, read out as a uniform value.
__device__ __forceinline__ uint32_t sum_before(const uint32_t* ws, int wave) {
  static_assert(kWaves == 16, "one total per lane of a 16-lane row");
  const int l = threadIdx.x & 15;
  uint32_t v = l < wave ? ws[l] : 0u;
  v += dpp<0x111, 0xf>(v);
  v += dpp<0x112, 0xf>(v);
  v += dpp<0x114, 0xf>(v);
  v += dpp<0x118, 0xf>(v);
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 15);
}

// Find the bin holding the k-th largest element (k >= 1) of a histogram of
// nb bins (4096 or 256) kept in NCOPY copies from h (stride kStride).
// Thread t owns a run of bins counted from the top, so a block-wide scan of
// the per-thread sums gives each run the number of elements above it.
// Returns via sh.bin / sh.above / sh.cnt.  CLEAR: once every copy has been
// read, zero copy 0 of sh.hist for the next pass.  All threads must call.
template <int NCOPY, bool CLEAR, int NC, int C>
__device__ void find_bin(Shared<NC, C>& sh, const uint32_t* h, int nb, uint32_t k) {
  constexpr int S = Shared<NC, C>::kStride;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t c4[4] = {0u, 0u, 0u, 0u};             // my bins, highest first
  int top;                                       // my highest bin
  int per;
  if (nb == 4 * kThreads) {                      // 4 bins: one 16-byte read per copy
    per = 4;
    top = nb - 1 - 4 * tid;
#pragma unroll
    for (int r = 0; r < NCOPY; ++r) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(&h[r * S + top - 3]);
      c4[0] += v.w;
      c4[1] += v.z;
      c4[2] += v.y;
      c4[3] += v.x;
    }
  } else {                                       // nb <= kThreads: one bin
    per = 1;
    top = nb - 1 - tid;
    if (top >= 0)
#pragma unroll
      for (int r = 0; r < NCOPY; ++r) c4[0] += h[r * S + top];
  }
  const uint32_t local = c4[0] + c4[1] + c4[2] + c4[3];
  const uint32_t incl = wave_incl_scan(local);
  if (lane == 63) sh.wsum[wave] = incl;
  __syncthreads();
  if constexpr (CLEAR) {
    for (int j = tid; j < kBins / 4; j += kThreads) st16(&sh.hist[4 * j], u32x4{0u, 0u, 0u, 0u});
  }
  uint32_t run = sum_before(sh.wsum, wave) + incl - local;   // count strictly above my bins
  if (run < k && run + local >= k) {
    for (int j = 0; j < per; ++j) {
      if (run + c4[j] >= k) {
        sh.bin = top - j;
        sh.above = run;
        sh.cnt = c4[j];
        break;
      }
      run += c4[j];
    }
  }
  __syncthreads();
}

// Selection of one row by the work-group (all threads call).  NC 16-byte
// chunks per thread kept in registers (0 = re-read each pass); C histogram
// copies.
template <int NC, int C>
__device__ __forceinline__ void topk_row(Shared<NC, C>& sh, const TopkLaunch& a, int row) {
  constexpr int S = Shared<NC, C>::kStride;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = row / a.q_count;
  const int i = a.q_begin + row % a.q_count;
  const int n_row = a.Lk - a.Lq + i + 1;          // visible keys of this query
  const int K = a.K;
  const float* src = a.scores + (int64_t)row * a.row_stride;
  const int n = n_row;                            // elements to select from
  int32_t* out = a.out + ((int64_t)b * a.Lq + i) * K;
  if (n <= K) {                                   // every visible position, then -1
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

  // Pass 1 histograms (C copies) and pass 3's small one start at zero.
  const uint32_t copy_base = (uint32_t)(lane & (C - 1)) * S;
  const uint32_t pad = (uint32_t)(iters * kThreads * 4 - n);
  auto clear_hists = [&]() {
    for (int j = tid; j < C * kBins / 4; j += kThreads) {
      const int r = j / (kBins / 4), o = j - r * (kBins / 4);
      st16(&sh.hist[r * S + 4 * o], u32x4{0u, 0u, 0u, 0u});
    }
    if (tid < 64) st16(&sh.h3[4 * tid], u32x4{0u, 0u, 0u, 0u});
    __syncthreads();
    if (tid == 0 && pad != 0u) atomicSub(&sh.hist[0], pad);
  };
  auto count1 = [&](const uint32_t (&kk)[4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) atomicAdd(&sh.hist[copy_base + (kk[e] >> 20)], 1u);
  };
  bool counted = false;                           // pass 1 already counted while loading

  uint32_t keys[NC > 0 ? NC : 1][4];
  if constexpr (NC > 0) {
    // Every load of the row is issued before any is converted, so the
    // chunks' latencies overlap and each conversion waits only for its own
    // chunk.  Chunks whole for every lane take one 16-byte load each, issued
    // unconditionally (chunks past the row re-read its first 16 bytes and
    // are masked): loads inside lane- or value-dependent branches would make
    // each chunk wait for the one before.  The ragged chunk (positions past
    // n read nothing) is loaded first, into registers of its own.
    const int cfull = a.vec_ok ? n / (4 * kThreads) : 0;
    const int crag = cfull < iters ? cfull : NC;  // the chunk loaded lane by lane
    auto inside = [&](int c, int e) { return c < cfull || (c < iters && (c * kThreads + tid) * 4 + e < n); };
    if (a.vec_ok && NC >= 8) {
      float vr[4] = {0.f, 0.f, 0.f, 0.f};        // the ragged chunk
      const int rpos = (crag * kThreads + tid) * 4;
      if (crag < NC) {
        // four clamped dword loads per lane, no lane-dependent branch (a
        // branch around a load makes the other path wait for it before it
        // writes the same registers, which serialised this load with the
        // rest); positions past n read the last score and are masked below
#pragma unroll
        for (int e = 0; e < 4; ++e) vr[e] = src[min(rpos + e, n - 1)];
      }
      float v[NC][4];
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const f32x4 t = *reinterpret_cast<const f32x4*>(src + (c < cfull ? (c * kThreads + tid) * 4 : 0));
        v[c][0] = t.x;
        v[c][1] = t.y;
        v[c][2] = t.z;
        v[c][3] = t.w;
      }
      // The histograms are cleared while the loads are in flight; each
      // chunk is then counted as soon as it has arrived (its conversion
      // waits for that chunk only), so pass 1 overlaps the row's transfer.
      clear_hists();
#pragma unroll
      for (int c = 0; c < NC; ++c) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          keys[c][e] = inside(c, e) ? order_key(c < cfull ? v[c][e] : vr[e]) : 0u;
        if (c < iters) count1(keys[c]);
      }
      counted = true;
    } else {
      // unaligned rows and short rows (one or two chunks: nothing to
      // overlap, and masked extra loads cost more than they hide): chunk by
      // chunk
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        if (c < iters) load_keys(c, keys[c]);
        else keys[c][0] = keys[c][1] = keys[c][2] = keys[c][3] = 0u;
      }
    }
  }

  // Radix passes.  prefix/mask describe the candidate set; k_rem counts how
  // many candidates are still to be taken (>= 1).
  //  - Pass 1 (bits 31..20) spreads its atomics over C histogram copies.
  //    Loaded slots past the row's end hold key 0; rows (not candidate
  //    lists) know how many there are, so pass 1 counts every slot, the
  //    padding into bin 0, and takes that many out of bin 0 again (atomics
  //    commute).
  //  - Later passes count one bin's elements, which the next bits spread
  //    thinly: one copy.  Pass 1's find step clears copy 0 for pass 2 once
  //    the copies are read, and pass 3 (bits 7..0) has a small histogram
  //    cleared at the start, so no pass has a clearing step of its own.
  uint32_t prefix = 0, mask = 0, k_rem = (uint32_t)K;
  bool whole = false;                             // the last bin is taken whole
  if (!counted) {
    clear_hists();
    if constexpr (NC > 0) {
#pragma unroll
      for (int c = 0; c < NC; ++c)
        if (c < iters) count1(keys[c]);
    } else {
      for (int c = 0; c < iters; ++c) {
        uint32_t kk[4];
        load_keys(c, kk);
        count1(kk);
      }
    }
  }
  {
    __syncthreads();
    find_bin<C, true>(sh, sh.hist, kBins, k_rem);
    const uint32_t cnt = sh.cnt;
    k_rem -= sh.above;
    prefix = sh.bin << 20;
    mask = 0xfff00000u;
    whole = cnt == k_rem;
  }
  if (!whole) {
    for (int pass = 1; pass < 3; ++pass) {
      const int sh_ = pass == 1 ? 8 : 0;
      const int nb = pass == 1 ? kBins : 256;
      uint32_t* const h = pass == 1 ? sh.hist : sh.h3;
      // prefix == 0 only if pass 1 chose bin 0; only then can padding match
      const bool check_pad = prefix == 0u;
      auto count = [&](const uint32_t (&kk)[4]) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if ((kk[e] & mask) == prefix && (!check_pad || kk[e] != 0u))
            atomicAdd(&h[(kk[e] >> sh_) & (nb - 1)], 1u);
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
      find_bin<1, false>(sh, h, nb, k_rem);
      const uint32_t cnt = sh.cnt;
      k_rem -= sh.above;
      prefix |= sh.bin << sh_;
      mask |= (uint32_t)(nb - 1) << sh_;
      if (cnt == k_rem) {                         // the whole bin is taken
        whole = true;
        break;
      }
    }
  }
  // hist is free from here on (the last find_bin ended with a barrier and
  // nothing reads it after): it becomes the output stage.
  const bool staged = K <= kBins;
  auto put = [&](uint32_t slot, int pos) {
    if (slot < (uint32_t)K) {                     // always, by construction
      if (staged) {
        sh.hist[slot] = (uint32_t)pos;
      } else {
        out[slot] = pos;
      }
    }
  };

  if constexpr (NC > 0) {
    // Bitmaps: chunk c of thread t covers positions 4*(c*kThreads + t) + e,
    // so the 8 lanes t = 8m..8m+7 fill word c*kThreads/8 + m, 4 bits each.
    // THR: one threshold, "above" = key > thr (no "equal" bitmap);
    // otherwise "above" and "equal" by prefix and mask.
    auto build_bits = [&](auto thr_tag, uint32_t thr) {
      constexpr bool THR = decltype(thr_tag)::value;
      const int sub = lane & 7;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        uint32_t gn = 0u, en = 0u;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t k = keys[c][e];
          if constexpr (THR) {
            gn |= k > thr ? (1u << e) : 0u;
          } else {
            const uint32_t m = k & mask;
            const bool valid = k != 0u;
            gn |= (valid && m > prefix) ? (1u << e) : 0u;
            en |= (valid && m == prefix) ? (1u << e) : 0u;
          }
        }
        // OR over lanes l-7..l: complete at lanes 7 and 15 of each DPP row
        uint32_t gw = gn << (4 * sub);
        gw |= dpp<0x111, 0xf>(gw);
        gw |= dpp<0x112, 0xf>(gw);
        gw |= dpp<0x114, 0xf>(gw);
        const int word = c * (kThreads / 8) + (tid >> 3);
        if (sub == 7) sh.gt_bits[word] = gw;
        if constexpr (!THR) {
          uint32_t ew = en << (4 * sub);
          ew |= dpp<0x111, 0xf>(ew);
          ew |= dpp<0x112, 0xf>(ew);
          ew |= dpp<0x114, 0xf>(ew);
          if (sub == 7) sh.eq_bits[word] = ew;
        }
      }
      __syncthreads();
    };
    // One thread per J consecutive words, in position order: a block-wide
    // scan of the word counts gives output slots; equal positions are taken
    // while fewer than k_rem came before (EQ).
    auto emit_words = [&](auto eq_tag) {
      constexpr bool EQ = decltype(eq_tag)::value;
      constexpr int W = Shared<NC, C>::kWords;
      constexpr int J = W >= kThreads ? W / kThreads : 1;
      const bool act = tid * J < W;
      uint32_t gw[J], ew[J], gc = 0u, ec = 0u;
#pragma unroll
      for (int j = 0; j < J; ++j) {
        gw[j] = act ? sh.gt_bits[tid * J + j] : 0u;
        ew[j] = (EQ && act) ? sh.eq_bits[tid * J + j] : 0u;
        gc += __builtin_popcount(gw[j]);
        if constexpr (EQ) ec += __builtin_popcount(ew[j]);
      }
      const uint32_t gi = wave_incl_scan(gc);
      const uint32_t ei = EQ ? wave_incl_scan(ec) : 0u;
      if (lane == 63) {
        sh.wsum[wave] = gi;
        if constexpr (EQ) sh.wsum[kWaves + wave] = ei;
      }
      __syncthreads();
      // counts before my first word
      uint32_t g_b = gi - gc + sum_before(sh.wsum, wave);
      uint32_t e_b = EQ ? ei - ec + sum_before(sh.wsum + kWaves, wave) : 0u;
#pragma unroll
      for (int j = 0; j < J; ++j) {
        uint32_t sel = gw[j];
        uint32_t slot = g_b;
        if constexpr (EQ) {
          uint32_t ek = ew[j];
          if (e_b >= k_rem) {
            ek = 0u;
          } else if (e_b + __builtin_popcount(ek) > k_rem) {
            uint32_t keep = 0u, rest = ek;
            for (uint32_t q = k_rem - e_b; q > 0u; --q) {
              const uint32_t low = rest & (0u - rest);
              keep |= low;
              rest ^= low;
            }
            ek = keep;
          }
          sel |= ek;
          slot += min(e_b, k_rem);
        }
        const int base = 32 * (tid * J + j);
        while (sel != 0u) {
          put(slot++, base + __builtin_ctz(sel));
          sel &= sel - 1u;
        }
        g_b += __builtin_popcount(gw[j]);
        if constexpr (EQ) e_b += __builtin_popcount(ew[j]);
      }
      __syncthreads();                            // the stage is complete
    };
    if (whole && prefix != 0u) {
      // the selection is key >= prefix (prefix != 0 excludes padding)
      build_bits(std::true_type{}, prefix - 1u);
      emit_words(std::false_type{});
    } else {
      build_bits(std::false_type{}, 0u);
      emit_words(std::true_type{});
    }
  } else {
    // Ordered emission: chunk c holds positions 4*(c*kThreads + tid) + 0..3,
    // so positions run over (chunk, thread, element).  A group of chunks is
    // scanned at once (one barrier): per chunk a block-wide exclusive scan of
    // the packed (gt, eq) counts, plus running totals over earlier chunks.
    uint32_t gt_run = 0, eq_run = 0;              // counts over earlier chunks
    auto emit_group = [&](int c0, int G, const uint32_t (*kk)[4]) {
      uint32_t packed[kGroup], incl[kGroup];
#pragma unroll
      for (int g = 0; g < kGroup; ++g) {
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
          incl[g] = wave_incl_scan(pk);
          if (lane == 63) sh.wsum[g * kWaves + wave] = incl[g];
        }
      }
      __syncthreads();
#pragma unroll
      for (int g = 0; g < kGroup; ++g) {
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
            if (gt || (eq && e_b < k_rem)) put(g_b + min(e_b, k_rem), pos0 + e);
            g_b += gt ? 1u : 0u;
            e_b += eq ? 1u : 0u;
          }
          gt_run += total & 0xffffu;
          eq_run += total >> 16;
        }
      }
      __syncthreads();                            // wsum is reused by the next group
    };
    for (int c0 = 0; c0 < iters; c0 += kGroup) {
      uint32_t kk[kGroup][4];
      const int G = min(kGroup, iters - c0);
#pragma unroll
      for (int g = 0; g < kGroup; ++g)
        if (g < G) load_keys(c0 + g, kk[g]);
      emit_group(c0, G, kk);
    }
  }
  // K' = min(K, n) = K here (n > K), so no padding is needed.
  if (staged) {
    if ((K & 3) == 0 && (reinterpret_cast<uintptr_t>(out) & 15u) == 0) {
      for (int j = tid; j < K / 4; j += kThreads)
        st16(out + 4 * j, u32x4{sh.hist[4 * j], sh.hist[4 * j + 1], sh.hist[4 * j + 2], sh.hist[4 * j + 3]});
    } else {
      for (int j = tid; j < K; j += kThreads) out[j] = (int32_t)sh.hist[j];
    }
  }
}

template <int NC, int C>
__global__ __launch_bounds__(kThreads, NC == 2 ? 8 : 4) void topk_kernel(TopkLaunch a) {
  __shared__ Shared<NC, C> sh;
  topk_row<NC, C>(sh, a, gridDim.x - 1 - blockIdx.x);   // longest rows first
}

// Filtered selection from the decode indexer's per-chunk candidate lists
// (see chunk_candidates in the indexer).  Thread t takes list slots 8t ..
// 8t + 7 of the row (chunk-major, so slot order is position order), keys 0
// past each list's count.  A radix select over the listed keys finds their
// K-th largest, T'.  When T''s 12-bit prefix lies above every chunk's cutoff
// bin, every key >= T' of the row is listed, so T' is the row's K-th largest
// key and the listed keys alone decide the selection; each thread then
// stores its chosen positions straight to their output slots (a few
// thousand 4-byte stores per row: staging them in LDS for 16-byte stores
// costs a barrier and measured slower).  Otherwise (or with fewer than K keys listed)
// the work-group selects from the full row of scores, NCF chunks per thread
// in registers.
template <int NCF>
__global__ __launch_bounds__(kThreads, 4) void topk_cand_kernel(TopkLaunch a) {
  constexpr int C = 8;
  __shared__ Shared<NCF, C> sh;
  __shared__ uint32_t s_total;
  __shared__ int s_cut;
  constexpr int S = Shared<NCF, C>::kStride;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = gridDim.x - 1 - blockIdx.x;
  const int b = row / a.q_count;
  const int i = a.q_begin + row % a.q_count;
  const int n = a.Lk - a.Lq + i + 1;
  const int K = a.K;
  int32_t* out = a.out + ((int64_t)b * a.Lq + i) * K;
  if (n <= K) {                                   // every visible position, then -1
    for (int j = tid; j < K; j += kThreads) out[j] = j < n ? j : -1;
    return;
  }
  const int M = a.cand_m, nch = a.cand_chunks;
  const int s0 = 8 * tid;                         // my first slot
  const bool act = s0 < nch * M;
  const int ch = act ? s0 / M : 0;
  const int sl = s0 - ch * M;                     // slot within the chunk's list
  const int64_t lst = (int64_t)row * nch + ch;
  uint32_t keys[2][4];
  uint32_t offs[4];
  int2 hd = int2{0, -1};
  if (act) {
    const u32x4 k0 = ld16(a.cand_keys + lst * kCandCap + sl);
    const u32x4 k1 = ld16(a.cand_keys + lst * kCandCap + sl + 4);
    const u32x4 o = ld16(a.cand_offs + lst * kCandCap + sl);
    hd = *reinterpret_cast<const int2*>(a.cand_hdr + 2 * lst);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      keys[0][e] = k0[e];
      keys[1][e] = k1[e];
      offs[e] = o[e];
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) keys[0][e] = keys[1][e] = offs[e] = 0u;
  }
  // pass 1 histograms (CC copies: a few thousand keys contend little), pass
  // 3's, and the two row-wide figures, cleared while the lists load
  constexpr int CC = 2;
  const uint32_t copy_base = (uint32_t)(lane & (CC - 1)) * S;
  for (int j = tid; j < CC * kBins / 4; j += kThreads) {
    const int r = j / (kBins / 4), o = j - r * (kBins / 4);
    st16(&sh.hist[r * S + 4 * o], u32x4{0u, 0u, 0u, 0u});
  }
  if (tid < 64) st16(&sh.h3[4 * tid], u32x4{0u, 0u, 0u, 0u});
  if (tid == 0) {
    s_total = 0u;
    s_cut = -1;
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (sl + 4 * c + e >= hd.x) keys[c][e] = 0u;
  uint32_t mine = 0u;
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (keys[c][e]) {
        atomicAdd(&sh.hist[copy_base + (keys[c][e] >> 20)], 1u);
        ++mine;
      }
  {
    const uint32_t incl = wave_incl_scan(mine);
    if (lane == 63 && incl) atomicAdd(&s_total, incl);
  }
  if (act && sl == 0 && hd.y >= 0) atomicMax(&s_cut, hd.y);   // one thread per chunk
  __syncthreads();
  const uint32_t total = s_total;
  const int cut = s_cut;
  bool ok = total >= (uint32_t)K;                 // uniform
  uint32_t prefix = 0, mask = 0, k_rem = (uint32_t)K;
  bool whole = false;
  if (ok) {
    find_bin<CC, true>(sh, sh.hist, kBins, k_rem);
    ok = (int)sh.bin > cut;
    const uint32_t cnt = sh.cnt;
    k_rem -= sh.above;
    prefix = sh.bin << 20;
    mask = 0xfff00000u;
    whole = cnt == k_rem;
  }
  if (!ok) {
    topk_row<NCF, C>(sh, a, row);                 // every thread takes this branch
    return;
  }
  if (!whole) {
    for (int pass = 1; pass < 3; ++pass) {
      const int sh_ = pass == 1 ? 8 : 0;
      const int nb = pass == 1 ? kBins : 256;
      uint32_t* const h = pass == 1 ? sh.hist : sh.h3;
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (keys[c][e] != 0u && (keys[c][e] & mask) == prefix)
            atomicAdd(&h[(keys[c][e] >> sh_) & (nb - 1)], 1u);
      __syncthreads();
      find_bin<1, false>(sh, h, nb, k_rem);
      const uint32_t cnt = sh.cnt;
      k_rem -= sh.above;
      prefix |= sh.bin << sh_;
      mask |= (uint32_t)(nb - 1) << sh_;
      if (cnt == k_rem) {                         // the whole bin is taken
        whole = true;
        break;
      }
    }
  }
  // Emission in slot (= position) order: a block-wide scan of each thread's
  // packed (above, equal) counts; equal keys are taken while fewer than
  // k_rem came before (all of them when the last bin is taken whole).
  const uint32_t quota = whole ? 0xffffffffu : k_rem;
  uint32_t pk = 0u;
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t k = keys[c][e], m = k & mask;
      pk += (k != 0u && m > prefix) ? 1u : 0u;
      pk += (k != 0u && m == prefix) ? 0x10000u : 0u;
    }
  const uint32_t incl = wave_incl_scan(pk);
  if (lane == 63) sh.wsum[wave] = incl;
  __syncthreads();
  const uint32_t excl = incl - pk + sum_before(sh.wsum, wave);
  uint32_t g_b = excl & 0xffffu, e_b = excl >> 16;
  const int pos0 = ch * kCandChunk;
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t k = keys[c][e], m = k & mask;
      const bool gt = k != 0u && m > prefix, eq = k != 0u && m == prefix;
      if (gt || (eq && e_b < quota)) {
        const uint32_t slot = g_b + min(e_b, quota);
        const int q = 4 * c + e;
        const int pos = pos0 + (int)((offs[q >> 1] >> (16 * (q & 1))) & 0xffffu);
        if (slot < (uint32_t)K) out[slot] = pos;  // always, by construction
      }
      g_b += gt ? 1u : 0u;
      e_b += eq ? 1u : 0u;
    }
}

}  // namespace

namespace {

void launch_rows(const TopkLaunch& a, int n_max, int grid, hipStream_t s) {
  const int chunks = (n_max + 3) / 4;
  const int iters = (chunks + kThreads - 1) / kThreads;
  // short rows come in large numbers (prefill): small histograms keep two
  // work-groups per CU; long rows are few and get the widest spreading.
  // Many rows of up to 32768 positions (long prefills) take 4 copies, which
  // fit two work-groups per CU (64K FP8 prefill: top-k 4.30 -> 3.96 ms per
  // step); a decode batch of such rows keeps 8.
  if (iters <= 2)
    launch_kernel(topk_kernel<2, 2>, dim3(grid), dim3(kThreads), 0, s, a);
  else if (iters <= 8 && grid >= 512)
    launch_kernel(topk_kernel<8, 4>, dim3(grid), dim3(kThreads), 0, s, a);
  else if (iters <= 8)
    launch_kernel(topk_kernel<8, 8>, dim3(grid), dim3(kThreads), 0, s, a);
  else if (iters <= 16)
    launch_kernel(topk_kernel<16, 8>, dim3(grid), dim3(kThreads), 0, s, a);
  else
    launch_kernel(topk_kernel<0, 8>, dim3(grid), dim3(kThreads), 0, s, a);
}

}  // namespace

int topk_cand_m(int n_max, int K) {
  // A chunk contributes about s = K / chunks of the chosen keys; with keys
  // spread evenly its count varies by about sqrt(s).  Lists get a margin of
  // 5 sqrt(s) + 16 keys over that share, so that their cutoff bins lie below
  // the K-th largest score of the row: with 16 chunks of 2048 keys (32768
  // positions) a chunk contributes about 128 keys and lists 256, a cutoff
  // several 12-bit bins (an eighth of an octave each) below it for index
  // scores.  A row whose chosen keys crowd into a few chunks falls back to
  // the full selection, and so does any row the margin does not cover.
  const int nch = (n_max + kCandChunk - 1) / kCandChunk;
  if (nch < 16 || K > kThreads * 4) return 0;
  int m = kCandMax / nch;
  m = (m < kCandCap ? m : kCandCap) & ~7;
  const double share = (double)K / nch;
  return (m >= 8 && m >= share + 5.0 * __builtin_sqrt(share) + 16.0) ? m : 0;
}

size_t topk_cand_bytes(int rows, int n_max) {
  const size_t lists = (size_t)rows * ((n_max + kCandChunk - 1) / kCandChunk);
  return lists * kCandCap * 4 + lists * kCandCap * 2 + lists * 8;
}

hipError_t launch_topk_cand(const TopkLaunch& a, hipStream_t s) {
  const int rows = a.B * a.q_count;
  const int n_max = a.Lk - a.Lq + a.q_begin + a.q_count;
  if (a.cand_m < 8 || (a.cand_m & 7) || a.cand_m > kCandCap || a.cand_chunks * a.cand_m > kCandMax ||
      a.cand_chunks != (a.Lk + kCandChunk - 1) / kCandChunk || a.K > kThreads * 4 || !a.cand_keys ||
      !a.cand_offs || !a.cand_hdr)
    return hipErrorInvalidValue;
  // the full-row fallback keeps rows of up to 65536 positions in registers
  const int iters = ((n_max + 3) / 4 + kThreads - 1) / kThreads;
  if (iters <= 8)
    launch_kernel(topk_cand_kernel<8>, dim3(rows), dim3(kThreads), 0, s, a);
  else if (iters <= 16)
    launch_kernel(topk_cand_kernel<16>, dim3(rows), dim3(kThreads), 0, s, a);
  else
    launch_kernel(topk_cand_kernel<0>, dim3(rows), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_topk(const TopkLaunch& a, hipStream_t s) {
  const int rows = a.B * a.q_count;
  const int n_max = a.Lk - a.Lq + a.q_begin + a.q_count;
  launch_rows(a, n_max, rows, s);
  return hipGetLastError();
}

}  // namespace dsa
