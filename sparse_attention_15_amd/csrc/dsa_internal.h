// Internal launch interface between the C-ABI front end (dsa_api.cpp) and
// the kernel translation units.  Host-only declarations.
#pragma once
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
};

struct TopkLaunch {
  const float* scores;     // rows as above
  int64_t row_stride;
  int32_t* out;            // row r at out + (b*Lq + i) * K  (full-tensor numbering)
  int B, Lq, Lk, K;
  int q_begin, q_count;
  int vec_ok;              // rows are 16-byte aligned: use 16-byte loads
  // two-stage selection (slices > 1): each row's slices of slice_len
  // positions first keep their own top K in cand [rows][slices][K]
  // (positions, -1 for none) with their scores in cand_score (same shape),
  // which the second stage reads in place of gathering them
  int slices, slice_len;
  int32_t* cand;
  float* cand_score;
};

struct AttnLaunch {
  const void* qa;          // [B][Lq][NH][Dqk]
  const void* kv;          // [B][Lc][Dqk]
  const int32_t* idx;      // [B][Lq][K] (full-tensor numbering)
  void* out;               // [B][Lq][NH][Dv]
  float* lse;              // [B][Lq][NH] or null
  void* part_o;            // split partials [rows][S][NH][Dv] (S > 1 only), in the
                           // output's precision: fp32 for fp32 out, bf16 for bf16 out
  float* part_lse;         // [rows][S][NH]
  int B, Lq, Lk, NH, Dqk, Dv, K;
  int Lc;                  // tokens per sequence in the latent cache (>= Lk)
  int q_begin, q_count;
  int splits;              // S: key ranges per query (1 = no combine step)
  float scale;
  int out_f32;             // out dtype: 1 fp32, 0 bf16
};

// Indexer.  *_bf16 / *_fp8 need H = 64, D = 128.
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
// Slices per row for a two-stage selection over `rows` rows of up to n_max
// positions (1 = single stage); writes the slice length.
int topk_slices(int rows, int n_max, int K, int* slice_len);

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

}  // namespace dsa
