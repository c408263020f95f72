// Internal launch interface between the C-ABI front end (dsa_api.cpp) and
// the kernel translation units.  Host-only declarations.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace dsa {

// Which queries of each sequence a launch covers: [q_begin, q_begin + q_count).
// Score rows and top-k rows of a launch are numbered r = b * q_count + (i - q_begin).
struct IndexLaunch {
  const void* q;           // [B][Lq][H][D] (bf16, f32 or fp8 codes)
  const uint8_t* q_scale;  // [B][Lq][H] ue8m0, fp8 only
  const void* k;           // [B][Lk][D]
  const uint8_t* k_scale;  // [B][Lk] ue8m0, fp8 only
  const float* w;          // [B][Lq][H]
  float* scores;           // rows of row_stride floats
  int64_t row_stride;
  int B, Lq, Lk, H, D;
  int Lc;                  // tokens per sequence in the key caches (>= Lk)
  int q_begin, q_count;
  int write_masked;        // also write -inf for positions beyond the causal limit
  uint32_t* zero_hist;     // decode shape only: rows x kTopkRowHeadWords words set to
                           // zero for the sliced top-k that follows (null: none)
  // Decode shape only: per-chunk candidate lists for the filtered top-k
  // (cand_m = 0: none).  Chunk c of a row covers keys [kCandChunk c,
  // kCandChunk (c + 1)); its list holds, in position order, every visible
  // key of the chunk whose 12-bit key prefix exceeds the chunk's cutoff bin
  // (at most cand_m of them; cutoff -1: every visible key).
  //   cand_keys [rows][chunks][kCandCap]  order keys
  //   cand_offs [rows][chunks][kCandCap]  positions within the chunk
  //   cand_hdr  [rows][chunks][2]         (count, cutoff bin)
  uint32_t* cand_keys;
  uint16_t* cand_offs;
  int32_t* cand_hdr;
  int cand_m;
};

// Candidate lists of the filtered decode top-k.
constexpr int kCandChunk = 2048;  // keys per list (the decode indexer's work-group chunk)
constexpr int kCandCap = 256;     // list slots per chunk
constexpr int kCandMax = 8192;    // candidate slots per row (chunks x cand_m)

struct TopkLaunch {
  const float* scores;     // rows as above
  int64_t row_stride;
  int32_t* out;            // row r at out + (b*Lq + i) * K  (full-tensor numbering)
  int B, Lq, Lk, K;
  int q_begin, q_count;
  int vec_ok;              // rows are 16-byte aligned: use 16-byte loads
  // sliced selection (launch_topk_sliced): rows cut into sl_count slices of
  // sl_len positions, one work-group each; workspace per row: a 4096-bin
  // histogram (zero on entry), per-slice counts [kMaxTopkSlices][2], the
  // row's threshold bin [4], per-slice kept lists of (key, position) and
  // per-slice candidate keys (those in the threshold bin)
  int sl_len, sl_count;
  uint32_t* sl_hist;
  int32_t* sl_info;
  int32_t* sl_rowinfo;
  uint32_t* sl_list;
  uint32_t* sl_cand;
  // filtered selection (launch_topk_cand): the decode indexer's candidate
  // lists (see IndexLaunch), cand_chunks per row, cand_m slots used per chunk
  const uint32_t* cand_keys;
  const uint16_t* cand_offs;
  const int32_t* cand_hdr;
  int cand_chunks, cand_m;
};

constexpr int kMaxTopkSlices = 512;
// Per-row head of the sliced top-k workspace, zero when a selection starts:
// a 4096-bin histogram followed by the row's barrier counters.
constexpr int kTopkRowHeadWords = 4096 + 64;

struct AttnLaunch {
  const void* qa;          // [B][Lq][NH][Dqk]
  const void* kv;          // [B][Lc][Dqk]
  const int32_t* idx;      // [B][Lq][K] (full-tensor numbering)
  void* out;               // [B][Lq][NH][Dv]
  float* lse;              // [B][Lq][NH] or null
  void* part_o;            // split partials, NH x Dv values per (row, split) (S > 1 only),
                           // in the output's precision (fp32 or bf16) and in the attention
                           // kernel's register order (see its epilogue)
  float* part_lse;         // [rows][S][NH]
  int B, Lq, Lk, NH, Dqk, Dv, K;
  int Lc;                  // tokens per sequence in the latent cache (>= Lk)
  int q_begin, q_count;
  int splits;              // S: key ranges per query (1 = no combine step)
  float scale;
  int out_f32;             // out dtype: 1 fp32, 0 bf16
};

// Indexer.  *_bf16 / *_fp8 need H = 64, D = 128.  Launches of at most
// kDecodeIndexQueries queries per sequence run the decode kernel, the only
// one that clears zero_hist (the others refuse it).
constexpr int kDecodeIndexQueries = 4;
hipError_t launch_index_f32(const IndexLaunch& a, hipStream_t s);
hipError_t launch_index_bf16(const IndexLaunch& a, hipStream_t s);
hipError_t launch_index_fp8(const IndexLaunch& a, hipStream_t s);

// Cache append: rows of n_new tokens per sequence copied to positions pos..
struct CacheAppend {
  int B, n_new, pos, cap;
  const void* k_new; const uint8_t* ks_new; const void* kv_new;
  void* k; uint8_t* ks; void* kv;
  int k_row_bytes, kv_row_bytes;
};
hipError_t launch_cache_append(const CacheAppend& c, hipStream_t s);

// FP8 producer: Hadamard rotation + ue8m0/E4M3 quantisation of 128-element rows.
hipError_t launch_rotate_quant(const void* x, int f32_in, int64_t rows, uint8_t* codes, uint8_t* scales,
                               hipStream_t s);

// Top-k (all dtypes: scores are fp32).
hipError_t launch_topk(const TopkLaunch& a, hipStream_t s);
// Sliced top-k for few long rows: slice length (1024, 2048 or 4096) for
// `rows` rows of up to n_max positions, or 0 when one work-group per row
// is the better plan; workspace bytes of that plan (and of its histogram,
// which must be zero when the selection starts).
int topk_sliced_len(int rows, int n_max, int K);
size_t topk_sliced_bytes(int rows, int n_max, int L, size_t* hist_bytes);
// zero_hist: clear the histogram first (else the caller's earlier kernel did).
hipError_t launch_topk_sliced(const TopkLaunch& a, bool zero_hist, hipStream_t s);
// Filtered top-k from the decode indexer's per-chunk candidate lists: list
// slots per chunk (cand_m) for rows of up to n_max positions, or 0 when the
// lists would not hold a safe margin over a chunk's share of the K chosen.
int topk_cand_m(int n_max, int K);
size_t topk_cand_bytes(int rows, int n_max);
hipError_t launch_topk_cand(const TopkLaunch& a, hipStream_t s);

// Sparse MLA.  *_bf16 needs NH = 128, Dqk = 576, Dv = 512.
hipError_t launch_attn_f32(const AttnLaunch& a, hipStream_t s);
hipError_t launch_attn_bf16(const AttnLaunch& a, hipStream_t s);
hipError_t launch_attn_combine(const AttnLaunch& a, hipStream_t s);

// C[m][n] = sum_k A[m][k] * B[n][k], bf16 in, fp32 accumulate; batch z adds
// z * s{a,b,c} elements to the bases.  K % 8 == 0, rows 16-byte aligned.
struct GemmLaunch {
  const uint16_t* A;
  const uint16_t* B;
  void* C;
  int M, N, K, batch;
  int64_t lda, ldb, ldc;   // row strides (elements)
  int64_t sa, sb, sc;      // batch strides (elements)
  int c_f32;               // 1: fp32 output, 0: bf16
  float* part;             // split-K partials [ksplit][batch][M][N] (ksplit > 1)
  int ksplit;              // 1: no split
};
hipError_t launch_gemm_bt(const GemmLaunch& g, hipStream_t s);
// Split count launch_gemm_bt would use for this shape given room for
// `avail` bytes of partials (1 = none); writes the bytes it needs.
int gemm_ksplit(int M, int N, int K, int batch, size_t* bytes);

// Split count the bf16 attention uses for a launch of `rows` queries.
int attn_splits_bf16(int rows, int K);

// Optional timing of a stage's launches, set by the timed forward on the
// launching host thread: the next launch records `start` as its kernel
// begins, and every launch records `stop` as its kernel ends, so the pair
// brackets the stage's kernels (no separate event packets between them).
struct StageEvents {
  hipEvent_t start, stop;
};
extern thread_local StageEvents g_stage_events;

// Every kernel of the path launches through here.
template <typename F, typename... Args>
inline void launch_kernel(F kernel, dim3 grid, dim3 block, size_t smem, hipStream_t s, Args... args) {
  StageEvents& ev = g_stage_events;
  if (ev.start || ev.stop) {
    hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)smem, s, ev.start, ev.stop, 0, args...);
    ev.start = nullptr;
  } else {
    hipLaunchKernelGGL(kernel, grid, block, smem, s, args...);
  }
}

}  // namespace dsa
