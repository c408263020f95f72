/*
 * dsa.h -- C ABI of the MI355X (gfx950) DeepSeek Sparse Attention hot path.
 *
 * The path has three steps, each exported on its own and fused in
 * dsa_forward:
 *   1. index scores  (lightning indexer: HF model doc "DeepSeek-V3.2",
 *      section "DeepSeek Sparse Attention (DSA)", item 1, and the paragraph on
 *      the single-head index-key cache that follows the list),
 *   2. per-query top-k selection (same section, item 2; index_topk in the
 *      released configuration excerpt of the atlas "DeepSeek-V3.2-Exp"
 *      token-ids page),
 *   3. sparse MLA attention in absorbed MQA form over the chosen latent rows
 *      (item 2; altools.ai "Technical Principles": MLA with MQA, key entries
 *      shared across query heads; visual-learn "DeepSeek-V3.2 / Exp",
 *      "Different questions select different tokens": the cache holds MLA's
 *      compressed vectors).
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is a caller-owned DEVICE pointer to a contiguous
 *     row-major array with the layout given below, 16-byte aligned.  The
 *     library never allocates, frees or keeps memory; temporary memory comes
 *     from a caller workspace sized by dsa_workspace_size().  The one
 *     exception is dsa_forward_static, which works in a fixed device array
 *     of the library (one per GPU) instead of a workspace.
 *   - Calls are asynchronous on `stream` (hipStream_t; 0 = the null stream):
 *     the caller keeps every buffer alive until the stream has passed the
 *     call.  No host synchronisation happens inside the library.
 *   - Argument checks run before any HIP call; on a failed check nothing is
 *     launched and the status says why.  Launch failures are reported as
 *     DSA_ERR_HIP.  No C++ exception crosses this interface.  After an error
 *     the contents of output buffers are undefined.
 *   - Query i of sequence b sits at position p = kv_len - q_len + i and sees
 *     keys 0..p (n = p + 1 of them): the causal mask keeps the diagonal
 *     (atlas token-ids page, transformer-forward excerpt), and a single decode
 *     query sees the whole cache.
 *   - The library keeps no mutable global state (dsa_forward_static's scratch
 *     array aside): calls on different streams or host threads are
 *     independent.
 */
#ifndef DSA_H_
#define DSA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSA_ABI_VERSION 6
#define DSA_MAX_KV_LEN_BF16 1864135   /* (2^31 - 1) / 1152 */

typedef enum {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARGUMENT = 1,   /* null pointer, bad size, misalignment */
  DSA_ERR_UNSUPPORTED = 2,        /* valid request this build has no kernel for */
  DSA_ERR_WORKSPACE_TOO_SMALL = 3,
  DSA_ERR_HIP = 4,                /* a HIP runtime call or launch failed */
  DSA_ERR_EXCEEDS_SCRATCH = 5     /* dsa_forward_static: the problem needs more
                                     than DSA_STATIC_SCRATCH_BYTES of scratch */
} dsa_status_t;

typedef enum {
  DSA_F32 = 0,
  DSA_BF16 = 1,
  DSA_FP8_E4M3 = 2                /* OCP E4M3 ("fn"): bias 7, max 448, no inf */
} dsa_dtype_t;

/* Problem description shared by all entry points. */
typedef struct {
  int32_t batch;        /* B sequences                                        */
  int32_t q_len;        /* Lq queries per sequence (1 for decode)             */
  int32_t kv_len;       /* Lk cached tokens per sequence, Lk >= Lq            */
  int32_t index_heads;  /* H index heads (index_n_heads, 64 in V3.2)          */
  int32_t index_dim;    /* D index head dim (index_head_dim, 128 in V3.2)     */
  int32_t topk;         /* K (index_topk, 2048 in V3.2)                       */
  int32_t attn_heads;   /* NH query heads of MLA (n_heads, 128 in V3.2)       */
  int32_t qk_dim;       /* Dqk = kv_lora_rank + qk_rope_head_dim (576)        */
  int32_t v_dim;        /* Dv = kv_lora_rank (512): values are the leading
                           Dv dims of each kv row (absorbed form)            */
  float softmax_scale;  /* multiplies q.k before the softmax                  */
  dsa_dtype_t index_dtype;  /* q_idx / k_idx element type                     */
  dsa_dtype_t attn_dtype;   /* q_attn / kv element type                       */
  dsa_dtype_t out_dtype;    /* out element type                               */
  int32_t kv_capacity;  /* tokens allocated per sequence in k_idx / k_scale / kv
                           (the sequence stride of the caches); 0 means
                           kv_len.  Must be 0 or >= kv_len.                  */
} dsa_problem_t;

/* Supported dtype combinations (anything else: DSA_ERR_UNSUPPORTED)
 *   index F32      + attn F32  + out F32         any dims within the limits below
 *   index BF16     + attn BF16 + out BF16|F32    H = 64, D = 128, NH = 128, Dqk = 576, Dv = 512
 *   index FP8_E4M3 + attn BF16 + out BF16|F32    same dims; q_scale/k_scale required
 * F32 limits: H*D <= 8192, Dqk <= 1024, Dv <= 1024, K <= 4096.
 * BF16 / FP8 limits: Lk <= DSA_MAX_KV_LEN_BF16 = 1864135 (latent rows are
 * gathered at byte offsets below 2^31 within a sequence: 1864135 rows of
 * 1152 bytes), K <= 65536.
 * All paths: K >= 1, Lq >= 1, Lk >= Lq, Lk <= 2^24 (scores rows in 32-bit indices).
 */

/* Step 1: index scores.
 *   Caches (k_idx, k_scale, kv) hold Lc = kv_capacity (or kv_len) tokens per
 *   sequence; only the first Lk are read.
 *   q_idx   [B][Lq][H][D]  index_dtype (FP8: E4M3 codes, one byte each)
 *   q_scale [B][Lq][H]     uint8 ue8m0 exponents, scale = 2^(e-127); FP8 only,
 *                          else NULL.  One scale per 128-element row.
 *   k_idx   [B][Lc][D]     index_dtype, the single-head index-key cache
 *   k_scale [B][Lc]        uint8 ue8m0 exponents; FP8 only, else NULL
 *   head_w  [B][Lq][H]     fp32 per-query head weights (any sign)
 *   scores  [B][Lq][Lk]    fp32 out:
 *       scores[b][i][s] = sum_h w[h] * max(0, q_h . k_s)   for s <= p
 *                       = -inf                              for s >  p
 *   With FP8 inputs q_h and k_s are the dequantised values code * scale;
 *   accumulation is fp32.
 */
dsa_status_t dsa_index_scores(const dsa_problem_t* prob,
                              const void* q_idx, const uint8_t* q_scale,
                              const void* k_idx, const uint8_t* k_scale,
                              const float* head_w, float* scores,
                              hipStream_t stream);

/* Step 2: exact per-row top-k.
 *   scores   fp32 rows, row (b, i) starts at scores + (b*Lq + i) * row_stride;
 *            only its first n = Lk - Lq + i + 1 entries are read.
 *            row_stride >= Lk (elements).  NaN inputs are not supported.
 *   topk_idx [B][Lq][K] int32 out: the K' = min(K, n) positions with the
 *            largest scores, larger score first and lower position first
 *            among equal scores (+0.0 == -0.0), written in ascending
 *            position order and padded with -1.  Bit-exact: the result is a
 *            pure function of the fp32 bit patterns.
 */
dsa_status_t dsa_topk(const dsa_problem_t* prob, const float* scores, int64_t row_stride,
                      int32_t* topk_idx, hipStream_t stream);

/* Step 2 with a workspace: the same result as dsa_topk, bit for bit.
 *   With few rows (B*Lq <= 128) of at least 4096 positions and more than K,
 *   each row is cut into slices of 1024-4096 positions, one work-group per
 *   slice, instead of one work-group per row; this needs
 *   dsa_workspace_size(prob, DSA_OP_TOPK) bytes of workspace (16-byte
 *   aligned).  When that size is 0 the call is dsa_topk (workspace may be
 *   NULL).  Too small a workspace: DSA_ERR_WORKSPACE_TOO_SMALL.
 */
dsa_status_t dsa_topk_ws(const dsa_problem_t* prob, const float* scores, int64_t row_stride,
                         int32_t* topk_idx, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Step 3: sparse MLA attention over the chosen rows (absorbed MQA form).
 *   q_attn   [B][Lq][NH][Dqk] attn_dtype
 *   kv       [B][Lc][Dqk]     attn_dtype; one latent row per token, shared
 *                             by all NH heads; values = its leading Dv dims
 *   topk_idx [B][Lq][K]       int32 positions; entries < 0 or >= Lk are
 *                             skipped, repeated entries count repeatedly; a
 *                             row with no usable entry gives out = 0 and
 *                             lse = -inf
 *   out      [B][Lq][NH][Dv]  out_dtype:
 *       out[a] = sum_j softmax_j(scale * q_a . kv_j) * kv_j[0:Dv] over chosen j
 *   lse      [B][Lq][NH] fp32 natural-log sum-exp of the scaled logits, or NULL
 *   workspace / workspace_bytes: at least dsa_workspace_size(prob, DSA_OP_ATTN)
 *            bytes (may be 0 bytes / NULL when that size is 0).
 */
dsa_status_t dsa_sparse_mla_attn(const dsa_problem_t* prob,
                                 const void* q_attn, const void* kv, const int32_t* topk_idx,
                                 void* out, float* lse,
                                 void* workspace, size_t workspace_bytes,
                                 hipStream_t stream);

/* Steps 1-3 fused in stream order (scores never leave the workspace).
 *   Tensors as above.  topk_idx may be NULL (then the indices live only in
 *   the workspace); if given it receives the selected positions.  lse may be
 *   NULL.  workspace: at least dsa_workspace_size(prob, DSA_OP_FORWARD) bytes.
 */
dsa_status_t dsa_forward(const dsa_problem_t* prob,
                         const void* q_idx, const uint8_t* q_scale,
                         const void* k_idx, const uint8_t* k_scale,
                         const float* head_w,
                         const void* q_attn, const void* kv,
                         int32_t* topk_idx, void* out, float* lse,
                         void* workspace, size_t workspace_bytes,
                         hipStream_t stream);

/* dsa_forward with per-kernel timing events (for measurement).
 *   events: n_events caller-created hipEvent_t handles, 2 per launch slot:
 *     events[2*(c*DSA_NUM_STAGES + s)] is recorded on `stream` before, and
 *     events[2*(c*DSA_NUM_STAGES + s) + 1] after, the launch of stage s for
 *     query chunk c, for every slot that fits in n_events.  Stages that do
 *     not run in a chunk record both events back to back.
 *   n_chunks_out: if not NULL, receives the number of query chunks used.
 */
#define DSA_NUM_STAGES 4   /* 0 indexer, 1 top-k, 2 attention, 3 split combine */
dsa_status_t dsa_forward_timed(const dsa_problem_t* prob,
                               const void* q_idx, const uint8_t* q_scale,
                               const void* k_idx, const uint8_t* k_scale,
                               const float* head_w,
                               const void* q_attn, const void* kv,
                               int32_t* topk_idx, void* out, float* lse,
                               void* workspace, size_t workspace_bytes,
                               hipEvent_t* events, int32_t n_events,
                               int32_t* n_chunks_out,
                               hipStream_t stream);

/* dsa_forward for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, results and launches as dsa_forward, but the workspace is
 * a static device array inside the library, DSA_STATIC_SCRATCH_BYTES large,
 * one per GPU: it is set up when the library's code is loaded on that GPU
 * and held until the process ends; the first call on a device looks up its
 * address there (hipGetSymbolAddress).  The call itself allocates nothing.
 *   The problem's forward workspace (dsa_workspace_size(prob,
 *   DSA_OP_FORWARD), less the top-k indices when topk_idx is given) must
 *   fit: else DSA_ERR_EXCEEDS_SCRATCH, before any HIP call.  Both decode
 *   shapes (32 x 32K and 8 x 128K) fit; long prefills do not.
 *   Runs on the current device, which must be the stream's.  Every call on
 *   one GPU works in that GPU's one array: calls whose stream work overlaps
 *   on one GPU (other streams, other host threads) race and give undefined
 *   results; calls in one stream's order are safe.  Nothing needs clearing
 *   between calls (every byte read is written earlier in the same call).
 */
#define DSA_STATIC_SCRATCH_BYTES ((size_t)96 << 20)
dsa_status_t dsa_forward_static(const dsa_problem_t* prob,
                                const void* q_idx, const uint8_t* q_scale,
                                const void* k_idx, const uint8_t* k_scale,
                                const float* head_w,
                                const void* q_attn, const void* kv,
                                int32_t* topk_idx, void* out, float* lse,
                                hipStream_t stream);

/* Cache append (HF doc "DeepSeek-V3.2", section "DeepSeek Sparse Attention
 * (DSA)": the indexer keeps its own cache of single-head index keys next to
 * the MLA cache, filled as tokens are processed; update_indexer in the usage
 * notes).  Writes n_new new tokens of every sequence into the caches at
 * positions kv_len .. kv_len + n_new - 1, so that a following call with
 * kv_len + n_new sees them.
 *   k_new       [B][n_new][D]    index_dtype
 *   k_new_scale [B][n_new]       uint8 ue8m0; FP8 index only, else NULL
 *   kv_new      [B][n_new][Dqk]  attn_dtype
 *   k_idx, k_scale, kv: the caches, [B][Lc][...] with Lc = kv_capacity,
 *   which must be >= kv_len + n_new (kv_capacity 0 is rejected here).
 *   Plain byte copies; n_new >= 0 (0 launches nothing).
 */
dsa_status_t dsa_cache_append(const dsa_problem_t* prob, int32_t n_new,
                              const void* k_new, const uint8_t* k_new_scale, const void* kv_new,
                              void* k_idx, uint8_t* k_scale, void* kv, hipStream_t stream);

/* FP8 producer of the index vectors (HF doc "DeepSeek-V3.2", section
 * "DeepSeek Sparse Attention (DSA)", item 1: the indexer runs in FP8 after an
 * orthogonal Hadamard rotation; "scale_fmt: ue8m0" in the released
 * configuration excerpt of the atlas "DeepSeek-V3.2-Exp" token-ids page).
 * Produces dsa_index_scores' FP8 inputs from bf16 / f32 activations: call it
 * once for the query rows ([B][Lq][H] rows) and once for the key rows
 * ([B][Lk] rows).
 *   x       [rows][dim] x_dtype (DSA_BF16 or DSA_F32), device
 *   codes   [rows][dim] uint8 out, device: E4M3 codes of y / 2^e
 *   scales  [rows] uint8 out, device: e + 127
 *   y = H x / sqrt(dim), H the Sylvester Hadamard matrix (H_1 = [1],
 *   H_2m = [[H_m, H_m], [H_m, -H_m]]), computed in fp32 as butterflies over
 *   strides 1, 2, ..., dim/2 followed by one multiply by fp32(1/sqrt(dim));
 *   e is the smallest integer with max|y| / 2^e <= 448 (0 for an all-zero
 *   row, clamped at -127); codes round to nearest, ties to even.
 *   dim must be 128 (else DSA_ERR_UNSUPPORTED); rows >= 0 (0 launches
 *   nothing); x 16-byte aligned, codes 8-byte aligned.
 */
dsa_status_t dsa_index_rotate_quantize(const void* x, dsa_dtype_t x_dtype, int64_t rows, int32_t dim,
                                       uint8_t* codes, uint8_t* scales, hipStream_t stream);

/* Projections on either side of the path (bf16 MFMA GEMMs, fp32 accumulation).
 * All operands bf16, row-major, 16-byte aligned; inner sizes multiples of 8.
 * Tokens are the B * Lq rows of the problem.
 *
 * Index query from the query latent (HF doc "DeepSeek-V3.2", usage notes:
 * the indexer scores queries from the low-rank query latent through its
 * wq_b projection, sized by q_lora_rank; q_lora_rank 1536, index_n_heads 64,
 * index_head_dim 128 in the released configuration excerpt, atlas token-ids
 * page):
 *   cq     [B][Lq][q_lora_rank]
 *   wq_b   [H*D][q_lora_rank]       output row h*D + d is head h, dim d
 *   q_idx  [B][Lq][H][D]            q_dtype: DSA_BF16 or DSA_F32
 *   q_idx[t][h][d] = sum_r cq[t][r] * wq_b[h*D + d][r].
 * For the FP8 index path, produce bf16 here and pass it to
 * dsa_index_rotate_quantize.
 */
dsa_status_t dsa_index_q_proj(const dsa_problem_t* prob, int32_t q_lora_rank, const void* cq, const void* wq_b,
                              void* q_idx, dsa_dtype_t q_dtype, hipStream_t stream);

/* Per-query head weights from the hidden state (the indexer's weights_proj,
 * kept out of FP8 in the usage example of the same doc; dim 7168 in the
 * configuration):
 *   x       [B][Lq][dim]
 *   w_proj  [H][dim]
 *   head_w  [B][Lq][H] fp32:  head_w[t][h] = sum_i x[t][i] * w_proj[h][i]
 * (no bias, no extra constant).
 *   workspace: optional (NULL, 0 allowed), 16-byte aligned, at least
 *   dsa_head_weights_workspace_size() bytes to be used: few-token calls then
 *   split the dim range over work-groups and add the partials in a fixed
 *   order (the result does not depend on whether the workspace is given
 *   beyond fp32 rounding of a different summation grouping).
 */
dsa_status_t dsa_head_weights_proj(const dsa_problem_t* prob, int32_t dim, const void* x, const void* w_proj,
                                   float* head_w, void* workspace, size_t workspace_bytes, hipStream_t stream);
size_t dsa_head_weights_workspace_size(const dsa_problem_t* prob, int32_t dim);

/* Un-absorption of the attention output: the value half of MLA's key/value
 * up-projection applied per head to the latent output (kv_lora_rank 512 and
 * v_head_dim 128 in the configuration):
 *   o_latent [B][Lq][NH][Dv]          dsa_sparse_mla_attn / dsa_forward output (bf16)
 *   w_uv     [NH][v_head_dim][Dv]
 *   out      [B][Lq][NH][v_head_dim]  out_dtype: DSA_BF16 or DSA_F32
 *   out[t][a][v] = sum_c o_latent[t][a][c] * w_uv[a][v][c].
 */
dsa_status_t dsa_out_unabsorb(const dsa_problem_t* prob, int32_t v_head_dim, const void* o_latent, const void* w_uv,
                              void* out, dsa_dtype_t out_dtype, hipStream_t stream);

#define DSA_OP_ATTN 1
#define DSA_OP_FORWARD 2
#define DSA_OP_TOPK 3
/* Workspace bytes needed by dsa_sparse_mla_attn (op = DSA_OP_ATTN),
 * dsa_forward (op = DSA_OP_FORWARD) or dsa_topk_ws (op = DSA_OP_TOPK) for
 * this problem; 0 for an invalid problem or op.  Pure host function, no HIP
 * call. */
size_t dsa_workspace_size(const dsa_problem_t* prob, int32_t op);

/* Number of query chunks dsa_forward splits this problem into (host only). */
int32_t dsa_forward_chunks(const dsa_problem_t* prob);

/* Number of work-groups each query's selected list is split over in
 * dsa_forward's attention step (1: no split, no combine launch); 0 for an
 * invalid problem.  Host only. */
int32_t dsa_forward_attn_splits(const dsa_problem_t* prob);

/* Positions per work-group of the sliced top-k dsa_forward uses for this
 * problem (1024, 2048 or 4096: each long decode row is cut into slices that
 * several work-groups select from together), or 0 when each row is selected
 * by one work-group (or the problem is invalid).  Host only. */
int32_t dsa_forward_topk_slice_len(const dsa_problem_t* prob);

/* List slots per 2048-key chunk of the filtered top-k dsa_forward uses for
 * this problem, or 0 when it selects from the full score rows (or the
 * problem is invalid).  Host only.  With decode-shaped launches of 16 or
 * more chunks per row, the indexer kernel also lists each chunk's
 * highest-scoring keys: every key whose 12-bit key prefix lies above a
 * cutoff bin that leaves at most this many keys.  The top-k then selects
 * from the lists alone whenever the K-th largest listed key lies above
 * every chunk's cutoff (then every key of the row at least as large is
 * listed); otherwise it selects from the full row.  The result is the
 * exact top-k either way (HF model doc "DeepSeek-V3.2", section "DeepSeek
 * Sparse Attention (DSA)", item 2: each query keeps its index_topk
 * best-scoring positions). */
int32_t dsa_forward_topk_list_slots(const dsa_problem_t* prob);

/* Static description of a status code. */
const char* dsa_status_string(dsa_status_t status);

/* DSA_ABI_VERSION of the built library. */
int32_t dsa_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* DSA_H_ */
