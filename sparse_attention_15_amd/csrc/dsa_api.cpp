// C-ABI front end of the DSA library: argument checks, workspace carving,
// query chunking and kernel dispatch.  No allocation, no host sync, no
// mutable global state.
#include "dsa.h"
#include "dsa_internal.h"

#include <atomic>
#include <cmath>
#include <cstdint>

using namespace dsa;

thread_local StageEvents dsa::g_stage_events = {nullptr, nullptr};

namespace {

constexpr size_t kAlign = 256;
constexpr size_t kScoresBudget = size_t(256) << 20;   // bytes of scores per query chunk
constexpr int64_t kMaxLk = int64_t(1) << 24;
// Row gathers address a sequence's latent rows with byte offsets below 2^31
// (1152-byte rows).
constexpr int64_t kMaxLkBf16 = DSA_MAX_KV_LEN_BF16;
static_assert(kMaxLkBf16 * 1152 <= (int64_t(1) << 31) - 1, "gather offsets stay below 2^31");

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool is_v32_dims_index(const dsa_problem_t& p) { return p.index_heads == 64 && p.index_dim == 128; }
bool is_v32_dims_attn(const dsa_problem_t& p) {
  return p.attn_heads == 128 && p.qk_dim == 576 && p.v_dim == 512;
}

enum Path { kPathF32, kPathBF16, kPathFP8 };

// Shape and dtype checks shared by every entry point.
dsa_status_t check_problem(const dsa_problem_t* p, Path* path) {
  if (!p) return DSA_ERR_INVALID_ARGUMENT;
  if (p->batch < 1 || p->q_len < 1 || p->kv_len < p->q_len || p->kv_len > kMaxLk) return DSA_ERR_INVALID_ARGUMENT;
  if (p->index_heads < 1 || p->index_dim < 1 || p->topk < 1) return DSA_ERR_INVALID_ARGUMENT;
  if (p->attn_heads < 1 || p->qk_dim < 1 || p->v_dim < 1 || p->v_dim > p->qk_dim) return DSA_ERR_INVALID_ARGUMENT;
  if (!std::isfinite(p->softmax_scale)) return DSA_ERR_INVALID_ARGUMENT;
  if (p->kv_capacity != 0 && p->kv_capacity < p->kv_len) return DSA_ERR_INVALID_ARGUMENT;
  const int it = p->index_dtype, at = p->attn_dtype, ot = p->out_dtype;
  if (it < DSA_F32 || it > DSA_FP8_E4M3 || at < DSA_F32 || at > DSA_FP8_E4M3 || ot < DSA_F32 || ot > DSA_FP8_E4M3)
    return DSA_ERR_INVALID_ARGUMENT;
  if (it == DSA_F32 && at == DSA_F32 && ot == DSA_F32) {
    if ((int64_t)p->index_heads * p->index_dim > 8192 || p->qk_dim > 1024 || p->v_dim > 1024 || p->topk > 4096)
      return DSA_ERR_UNSUPPORTED;
    *path = kPathF32;
    return DSA_OK;
  }
  if ((it == DSA_BF16 || it == DSA_FP8_E4M3) && at == DSA_BF16 && (ot == DSA_BF16 || ot == DSA_F32)) {
    if (!is_v32_dims_index(*p) || !is_v32_dims_attn(*p) || p->kv_len > kMaxLkBf16 || p->topk > 65536)
      return DSA_ERR_UNSUPPORTED;
    *path = it == DSA_BF16 ? kPathBF16 : kPathFP8;
    return DSA_OK;
  }
  return DSA_ERR_UNSUPPORTED;
}

dsa_status_t hip_status(hipError_t e) { return e == hipSuccess ? DSA_OK : DSA_ERR_HIP; }

int chunk_queries(const dsa_problem_t& p) {
  const int64_t row_bytes = (int64_t)p.kv_len * 4 * p.batch;
  int64_t cq = (int64_t)kScoresBudget / row_bytes;
  if (cq >= p.q_len) return p.q_len;
  if (cq >= 8) cq = cq / 8 * 8;
  return (int)(cq < 1 ? 1 : cq);
}

int attn_splits(const dsa_problem_t& p, Path path, int rows) {
  return path == kPathF32 ? 1 : attn_splits_bf16(rows, p.topk);
}

size_t attn_partials_bytes(const dsa_problem_t& p, int rows, int splits) {
  if (splits <= 1) return 0;
  return align_up((size_t)rows * splits * p.attn_heads * p.v_dim * 4) +
         align_up((size_t)rows * splits * p.attn_heads * 4);
}

struct ForwardPlan {
  int chunk;       // queries per chunk
  int n_chunks;
  int tk_sl_len;                 // sliced top-k: positions per work-group (0 = not used)
  int tk_cand_m;                 // filtered top-k: list slots per chunk (0 = not used)
  size_t scores_bytes, idx_bytes, part_bytes, cand_bytes;
  size_t total() const { return scores_bytes + idx_bytes + part_bytes + cand_bytes; }
};

ForwardPlan plan_forward(const dsa_problem_t& p, Path path, bool need_idx) {
  ForwardPlan f;
  f.chunk = chunk_queries(p);
  f.n_chunks = (p.q_len + f.chunk - 1) / f.chunk;
  f.scores_bytes = align_up((size_t)p.batch * f.chunk * p.kv_len * 4);
  f.idx_bytes = need_idx ? align_up((size_t)p.batch * p.q_len * p.topk * 4) : 0;
  const int rows = p.batch * f.chunk;
  f.part_bytes = attn_partials_bytes(p, rows, attn_splits(p, path, rows));
  // Decode-shaped rows (the decode indexer kernel runs): with enough
  // 2048-key chunks the indexer lists each chunk's candidates and top-k
  // selects from the lists; else few long rows take one work-group per row
  // slice (the decode indexer zeroes the histogram the sliced selection
  // accumulates into).
  const bool decode = path != kPathF32 && f.chunk <= kDecodeIndexQueries;
  f.tk_cand_m = decode ? topk_cand_m(p.kv_len, p.topk) : 0;
  f.tk_sl_len = (decode && f.tk_cand_m == 0) ? topk_sliced_len(rows, p.kv_len, p.topk) : 0;
  f.cand_bytes = 0;
  if (f.tk_cand_m > 0) {
    f.cand_bytes = align_up(topk_cand_bytes(rows, p.kv_len));
  } else if (f.tk_sl_len > 0) {
    size_t hist_bytes;
    f.cand_bytes = align_up(topk_sliced_bytes(rows, p.kv_len, f.tk_sl_len, &hist_bytes));
  }
  return f;
}

// Workspace pieces of the sliced top-k, in the order topk_sliced_bytes counts them.
void carve_sliced(TopkLaunch& ta, char* base, int rows, int n_max, int L) {
  size_t hist_bytes;
  topk_sliced_bytes(rows, n_max, L, &hist_bytes);
  ta.sl_len = L;
  ta.sl_count = (n_max + L - 1) / L;
  ta.sl_hist = reinterpret_cast<uint32_t*>(base);
  ta.sl_info = reinterpret_cast<int32_t*>(base + hist_bytes);
  ta.sl_rowinfo = ta.sl_info + (size_t)rows * kMaxTopkSlices * 2;
  ta.sl_list = reinterpret_cast<uint32_t*>(ta.sl_rowinfo + (size_t)rows * 4);
  ta.sl_cand = ta.sl_list + (size_t)rows * ta.sl_count * L * 2;
}

// Workspace pieces of the filtered top-k's candidate lists, in the order
// topk_cand_bytes counts them: keys, positions within the chunk, headers.
void carve_cand(IndexLaunch& ia, TopkLaunch& ta, char* base, int rows, int n_max, int m) {
  const int nch = (n_max + kCandChunk - 1) / kCandChunk;
  const size_t lists = (size_t)rows * nch;
  ia.cand_keys = reinterpret_cast<uint32_t*>(base);
  ia.cand_offs = reinterpret_cast<uint16_t*>(base + lists * kCandCap * 4);
  ia.cand_hdr = reinterpret_cast<int32_t*>(base + lists * kCandCap * 6);
  ia.cand_m = m;
  ta.cand_keys = ia.cand_keys;
  ta.cand_offs = ia.cand_offs;
  ta.cand_hdr = ia.cand_hdr;
  ta.cand_chunks = nch;
  ta.cand_m = m;
}

IndexLaunch make_index(const dsa_problem_t& p, const void* q, const uint8_t* qs, const void* k, const uint8_t* ks,
                       const float* w, float* scores, int64_t row_stride, int q_begin, int q_count, int masked) {
  IndexLaunch a;
  a.q = q; a.q_scale = qs; a.k = k; a.k_scale = ks; a.w = w;
  a.scores = scores; a.row_stride = row_stride;
  a.B = p.batch; a.Lq = p.q_len; a.Lk = p.kv_len; a.H = p.index_heads; a.D = p.index_dim;
  a.Lc = p.kv_capacity ? p.kv_capacity : p.kv_len;
  a.q_begin = q_begin; a.q_count = q_count; a.write_masked = masked;
  a.zero_hist = nullptr;
  a.cand_keys = nullptr; a.cand_offs = nullptr; a.cand_hdr = nullptr; a.cand_m = 0;
  return a;
}

TopkLaunch make_topk(const dsa_problem_t& p, const float* scores, int64_t row_stride, int32_t* out,
                     int q_begin, int q_count) {
  TopkLaunch a;
  a.scores = scores; a.row_stride = row_stride; a.out = out;
  a.B = p.batch; a.Lq = p.q_len; a.Lk = p.kv_len; a.K = p.topk;
  a.q_begin = q_begin; a.q_count = q_count;
  a.vec_ok = aligned16(scores) && (row_stride % 4) == 0;
  a.sl_len = 0; a.sl_count = 0; a.sl_hist = nullptr; a.sl_info = nullptr; a.sl_rowinfo = nullptr;
  a.sl_list = nullptr; a.sl_cand = nullptr;
  a.cand_keys = nullptr; a.cand_offs = nullptr; a.cand_hdr = nullptr; a.cand_chunks = 0; a.cand_m = 0;
  return a;
}

AttnLaunch make_attn(const dsa_problem_t& p, const void* qa, const void* kv, const int32_t* idx, void* out,
                     float* lse, int q_begin, int q_count, int splits, void* part) {
  AttnLaunch a;
  a.qa = qa; a.kv = kv; a.idx = idx; a.out = out; a.lse = lse;
  a.B = p.batch; a.Lq = p.q_len; a.Lk = p.kv_len; a.NH = p.attn_heads; a.Dqk = p.qk_dim; a.Dv = p.v_dim;
  a.Lc = p.kv_capacity ? p.kv_capacity : p.kv_len;
  a.K = p.topk; a.q_begin = q_begin; a.q_count = q_count; a.splits = splits;
  a.scale = p.softmax_scale; a.out_f32 = p.out_dtype == DSA_F32;
  a.part_o = nullptr; a.part_lse = nullptr;
  if (splits > 1) {
    const int rows = p.batch * q_count;
    a.part_o = part;
    a.part_lse = reinterpret_cast<float*>(static_cast<char*>(part) +
                                          align_up((size_t)rows * splits * p.attn_heads * p.v_dim * 4));
  }
  return a;
}

hipError_t run_index(Path path, const IndexLaunch& a, hipStream_t s) {
  if (path == kPathF32) return launch_index_f32(a, s);
  if (path == kPathBF16) return launch_index_bf16(a, s);
  return launch_index_fp8(a, s);
}

dsa_status_t check_index_ptrs(Path path, const void* q, const uint8_t* qs, const void* k, const uint8_t* ks,
                              const float* w) {
  if (!q || !k || !w) return DSA_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k) || !aligned16(w)) return DSA_ERR_INVALID_ARGUMENT;
  if (path == kPathFP8 && (!qs || !ks)) return DSA_ERR_INVALID_ARGUMENT;
  return DSA_OK;
}

dsa_status_t check_attn_ptrs(const void* qa, const void* kv, const void* out) {
  if (!qa || !kv || !out) return DSA_ERR_INVALID_ARGUMENT;
  if (!aligned16(qa) || !aligned16(kv) || !aligned16(out)) return DSA_ERR_INVALID_ARGUMENT;
  return DSA_OK;
}

// Times stage `stage` of chunk `chunk` with events[slot*2], events[slot*2+1]
// if that slot exists: rec(.., 0) attaches them to the stage's launches (the
// first kernel's start, the last kernel's end); rec(.., 1) records both by
// themselves if the stage launched nothing.
struct EventSink {
  hipEvent_t* ev;
  int n_slots;
  hipStream_t s;
  hipError_t rec(int chunk, int stage, int which) const {
    const int slot = chunk * DSA_NUM_STAGES + stage;
    if (!ev || slot >= n_slots) return hipSuccess;
    if (which == 0) {
      g_stage_events = StageEvents{ev[2 * slot], ev[2 * slot + 1]};
      return hipSuccess;
    }
    hipError_t e = hipSuccess;
    if (g_stage_events.start) {                   // nothing was launched
      if ((e = hipEventRecord(ev[2 * slot], s)) == hipSuccess) e = hipEventRecord(ev[2 * slot + 1], s);
    }
    g_stage_events = StageEvents{nullptr, nullptr};
    return e;
  }
};

dsa_status_t forward_impl(const dsa_problem_t* prob, const void* q_idx, const uint8_t* q_scale, const void* k_idx,
                          const uint8_t* k_scale, const float* head_w, const void* q_attn, const void* kv,
                          int32_t* topk_idx, void* out, float* lse, void* workspace, size_t workspace_bytes,
                          const EventSink& ev, int32_t* n_chunks_out, hipStream_t stream) {
  struct StageReset {                             // no stage timing outlives the call, on any return
    ~StageReset() { g_stage_events = StageEvents{nullptr, nullptr}; }
  } stage_reset;
  Path path;
  dsa_status_t st = check_problem(prob, &path);
  if (st != DSA_OK) return st;
  const dsa_problem_t& p = *prob;
  if ((st = check_index_ptrs(path, q_idx, q_scale, k_idx, k_scale, head_w)) != DSA_OK) return st;
  if ((st = check_attn_ptrs(q_attn, kv, out)) != DSA_OK) return st;
  if ((topk_idx && !aligned16(topk_idx)) || (lse && !aligned16(lse))) return DSA_ERR_INVALID_ARGUMENT;
  const ForwardPlan f = plan_forward(p, path, topk_idx == nullptr);
  const size_t need = f.total();
  if (workspace_bytes < need) return DSA_ERR_WORKSPACE_TOO_SMALL;
  if (!workspace || !aligned16(workspace)) return DSA_ERR_INVALID_ARGUMENT;
  if (n_chunks_out) *n_chunks_out = f.n_chunks;

  char* ws = static_cast<char*>(workspace);
  float* scores = reinterpret_cast<float*>(ws);
  int32_t* idx = topk_idx ? topk_idx : reinterpret_cast<int32_t*>(ws + f.scores_bytes);
  void* part = ws + f.scores_bytes + f.idx_bytes;
  int32_t* cand = reinterpret_cast<int32_t*>(ws + f.scores_bytes + f.idx_bytes + f.part_bytes);

  for (int c = 0; c < f.n_chunks; ++c) {
    const int q0 = c * f.chunk;
    const int qn = p.q_len - q0 < f.chunk ? p.q_len - q0 : f.chunk;
    hipError_t e;
    // 1. scores for this chunk's rows (causal part only)
    if ((e = ev.rec(c, 0, 0)) != hipSuccess) return DSA_ERR_HIP;
    IndexLaunch ia = make_index(p, q_idx, q_scale, k_idx, k_scale, head_w, scores, p.kv_len, q0, qn, 0);
    TopkLaunch ta = make_topk(p, scores, p.kv_len, idx, q0, qn);
    if (f.tk_cand_m > 0) {
      carve_cand(ia, ta, reinterpret_cast<char*>(cand), p.batch * f.chunk, p.kv_len, f.tk_cand_m);
    } else if (f.tk_sl_len > 0) {
      carve_sliced(ta, reinterpret_cast<char*>(cand), p.batch * f.chunk, p.kv_len, f.tk_sl_len);
      ia.zero_hist = ta.sl_hist;
    }
    if ((e = run_index(path, ia, stream)) != hipSuccess) return hip_status(e);
    if ((e = ev.rec(c, 0, 1)) != hipSuccess) return DSA_ERR_HIP;
    // 2. top-k
    if ((e = ev.rec(c, 1, 0)) != hipSuccess) return DSA_ERR_HIP;
    e = f.tk_cand_m > 0   ? launch_topk_cand(ta, stream)
        : f.tk_sl_len > 0 ? launch_topk_sliced(ta, false, stream)
                          : launch_topk(ta, stream);
    if (e != hipSuccess) return hip_status(e);
    if ((e = ev.rec(c, 1, 1)) != hipSuccess) return DSA_ERR_HIP;
    // 3. attention (+ combine); every chunk uses the split count the
    //    workspace was sized for (that of a full chunk)
    const int splits = attn_splits(p, path, p.batch * f.chunk);
    AttnLaunch aa = make_attn(p, q_attn, kv, idx, out, lse, q0, qn, splits, part);
    if ((e = ev.rec(c, 2, 0)) != hipSuccess) return DSA_ERR_HIP;
    e = path == kPathF32 ? launch_attn_f32(aa, stream) : launch_attn_bf16(aa, stream);
    if (e != hipSuccess) return hip_status(e);
    if ((e = ev.rec(c, 2, 1)) != hipSuccess) return DSA_ERR_HIP;
    if ((e = ev.rec(c, 3, 0)) != hipSuccess) return DSA_ERR_HIP;
    if (splits > 1 && (e = launch_attn_combine(aa, stream)) != hipSuccess) return hip_status(e);
    if ((e = ev.rec(c, 3, 1)) != hipSuccess) return DSA_ERR_HIP;
  }
  return DSA_OK;
}

// Shared checks of the projections: bf16 operands with 16-byte rows.
dsa_status_t run_gemm(const void* a, const void* b, void* c, int m, int n, int k, int batch, int64_t lda,
                      int64_t ldb, int64_t ldc, int64_t sa, int64_t sb, int64_t sc, dsa_dtype_t c_dtype,
                      hipStream_t stream, void* workspace = nullptr, size_t workspace_bytes = 0) {
  if (!a || !b || !c || k < 8 || (k & 7) || (lda & 7) || (ldb & 7)) return DSA_ERR_INVALID_ARGUMENT;
  if (c_dtype != DSA_BF16 && c_dtype != DSA_F32) return DSA_ERR_INVALID_ARGUMENT;
  if (!aligned16(a) || !aligned16(b) || (reinterpret_cast<uintptr_t>(c) & 3u)) return DSA_ERR_INVALID_ARGUMENT;
  GemmLaunch g;
  g.A = static_cast<const uint16_t*>(a);
  g.B = static_cast<const uint16_t*>(b);
  g.C = c;
  g.M = m; g.N = n; g.K = k; g.batch = batch;
  g.lda = lda; g.ldb = ldb; g.ldc = ldc;
  g.sa = sa; g.sb = sb; g.sc = sc;
  g.c_f32 = c_dtype == DSA_F32;
  g.part = nullptr;
  g.ksplit = 1;
  size_t need = 0;
  const int ks = gemm_ksplit(m, n, k, batch, &need);
  if (ks > 1 && workspace && workspace_bytes >= need && aligned16(workspace)) {
    g.part = static_cast<float*>(workspace);
    g.ksplit = ks;
  }
  return hip_status(launch_gemm_bt(g, stream));
}

}  // namespace

extern "C" {

dsa_status_t dsa_index_scores(const dsa_problem_t* prob, const void* q_idx, const uint8_t* q_scale,
                              const void* k_idx, const uint8_t* k_scale, const float* head_w, float* scores,
                              hipStream_t stream) {
  Path path;
  dsa_status_t st = check_problem(prob, &path);
  if (st != DSA_OK) return st;
  if ((st = check_index_ptrs(path, q_idx, q_scale, k_idx, k_scale, head_w)) != DSA_OK) return st;
  if (!scores || !aligned16(scores)) return DSA_ERR_INVALID_ARGUMENT;
  const dsa_problem_t& p = *prob;
  IndexLaunch a = make_index(p, q_idx, q_scale, k_idx, k_scale, head_w, scores, p.kv_len, 0, p.q_len, 1);
  return hip_status(run_index(path, a, stream));
}

dsa_status_t dsa_topk(const dsa_problem_t* prob, const float* scores, int64_t row_stride, int32_t* topk_idx,
                      hipStream_t stream) {
  Path path;
  dsa_status_t st = check_problem(prob, &path);
  if (st != DSA_OK) return st;
  if (!scores || !topk_idx || row_stride < prob->kv_len) return DSA_ERR_INVALID_ARGUMENT;
  if ((reinterpret_cast<uintptr_t>(scores) & 3u) || (reinterpret_cast<uintptr_t>(topk_idx) & 3u))
    return DSA_ERR_INVALID_ARGUMENT;
  return hip_status(launch_topk(make_topk(*prob, scores, row_stride, topk_idx, 0, prob->q_len), stream));
}

dsa_status_t dsa_topk_ws(const dsa_problem_t* prob, const float* scores, int64_t row_stride, int32_t* topk_idx,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
  Path path;
  dsa_status_t st = check_problem(prob, &path);
  if (st != DSA_OK) return st;
  if (!scores || !topk_idx || row_stride < prob->kv_len) return DSA_ERR_INVALID_ARGUMENT;
  if ((reinterpret_cast<uintptr_t>(scores) & 3u) || (reinterpret_cast<uintptr_t>(topk_idx) & 3u))
    return DSA_ERR_INVALID_ARGUMENT;
  const dsa_problem_t& p = *prob;
  TopkLaunch ta = make_topk(p, scores, row_stride, topk_idx, 0, p.q_len);
  const int rows = p.batch * p.q_len;
  const int L = topk_sliced_len(rows, p.kv_len, p.topk);
  if (L == 0) return hip_status(launch_topk(ta, stream));
  size_t hist_bytes;
  if (workspace_bytes < topk_sliced_bytes(rows, p.kv_len, L, &hist_bytes)) return DSA_ERR_WORKSPACE_TOO_SMALL;
  if (!workspace || !aligned16(workspace)) return DSA_ERR_INVALID_ARGUMENT;
  carve_sliced(ta, static_cast<char*>(workspace), rows, p.kv_len, L);
  return hip_status(launch_topk_sliced(ta, true, stream));
}

dsa_status_t dsa_sparse_mla_attn(const dsa_problem_t* prob, const void* q_attn, const void* kv,
                                 const int32_t* topk_idx, void* out, float* lse, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  Path path;
  dsa_status_t st = check_problem(prob, &path);
  if (st != DSA_OK) return st;
  if ((st = check_attn_ptrs(q_attn, kv, out)) != DSA_OK) return st;
  if (!topk_idx || !aligned16(topk_idx) || (lse && !aligned16(lse))) return DSA_ERR_INVALID_ARGUMENT;
  const dsa_problem_t& p = *prob;
  const int rows = p.batch * p.q_len;
  const int splits = attn_splits(p, path, rows);
  const size_t need = attn_partials_bytes(p, rows, splits);
  if (workspace_bytes < need) return DSA_ERR_WORKSPACE_TOO_SMALL;
  if (need > 0 && (!workspace || !aligned16(workspace))) return DSA_ERR_INVALID_ARGUMENT;
  AttnLaunch a = make_attn(p, q_attn, kv, topk_idx, out, lse, 0, p.q_len, splits, workspace);
  hipError_t e = path == kPathF32 ? launch_attn_f32(a, stream) : launch_attn_bf16(a, stream);
  if (e != hipSuccess) return hip_status(e);
  if (splits > 1) return hip_status(launch_attn_combine(a, stream));
  return DSA_OK;
}

dsa_status_t dsa_forward(const dsa_problem_t* prob, const void* q_idx, const uint8_t* q_scale, const void* k_idx,
                         const uint8_t* k_scale, const float* head_w, const void* q_attn, const void* kv,
                         int32_t* topk_idx, void* out, float* lse, void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
  EventSink none{nullptr, 0, stream};
  return forward_impl(prob, q_idx, q_scale, k_idx, k_scale, head_w, q_attn, kv, topk_idx, out, lse, workspace,
                      workspace_bytes, none, nullptr, stream);
}

dsa_status_t dsa_forward_timed(const dsa_problem_t* prob, const void* q_idx, const uint8_t* q_scale,
                               const void* k_idx, const uint8_t* k_scale, const float* head_w, const void* q_attn,
                               const void* kv, int32_t* topk_idx, void* out, float* lse, void* workspace,
                               size_t workspace_bytes, hipEvent_t* events, int32_t n_events,
                               int32_t* n_chunks_out, hipStream_t stream) {
  if (n_events < 0 || (n_events > 0 && !events)) return DSA_ERR_INVALID_ARGUMENT;
  EventSink sink{events, n_events / 2, stream};
  return forward_impl(prob, q_idx, q_scale, k_idx, k_scale, head_w, q_attn, kv, topk_idx, out, lse, workspace,
                      workspace_bytes, sink, n_chunks_out, stream);
}

// ------------------------------------------------------ allocation-free ---
namespace {

// dsa_forward_static's workspace: one copy of this array per GPU, created
// when the code object is loaded there and kept until the process ends.  In
// host code the name only stands for the symbol; kernels get the device
// address hipGetSymbolAddress gives for the current GPU.
static __device__ __align__(256) unsigned char scratch[DSA_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];

// Device address of the current GPU's scratch array, looked up on the first
// call on that device (null if the device or the lookup fails).
void* static_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (p) return p;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
  g_scratch_addr[dev].store(p, std::memory_order_release);
  return p;
}

}  // namespace

dsa_status_t dsa_forward_static(const dsa_problem_t* prob, const void* q_idx, const uint8_t* q_scale,
                                const void* k_idx, const uint8_t* k_scale, const float* head_w,
                                const void* q_attn, const void* kv, int32_t* topk_idx, void* out, float* lse,
                                hipStream_t stream) {
  // every argument check before the first HIP call
  Path path;
  dsa_status_t st = check_problem(prob, &path);
  if (st != DSA_OK) return st;
  if ((st = check_index_ptrs(path, q_idx, q_scale, k_idx, k_scale, head_w)) != DSA_OK) return st;
  if ((st = check_attn_ptrs(q_attn, kv, out)) != DSA_OK) return st;
  if ((topk_idx && !aligned16(topk_idx)) || (lse && !aligned16(lse))) return DSA_ERR_INVALID_ARGUMENT;
  if (plan_forward(*prob, path, topk_idx == nullptr).total() > DSA_STATIC_SCRATCH_BYTES)
    return DSA_ERR_EXCEEDS_SCRATCH;
  void* ws = static_scratch();
  if (!ws) return DSA_ERR_HIP;
  EventSink none{nullptr, 0, stream};
  return forward_impl(prob, q_idx, q_scale, k_idx, k_scale, head_w, q_attn, kv, topk_idx, out, lse, ws,
                      DSA_STATIC_SCRATCH_BYTES, none, nullptr, stream);
}

size_t dsa_workspace_size(const dsa_problem_t* prob, int32_t op) {
  Path path;
  if (check_problem(prob, &path) != DSA_OK) return 0;
  const dsa_problem_t& p = *prob;
  if (op == DSA_OP_ATTN) {
    const int rows = p.batch * p.q_len;
    return attn_partials_bytes(p, rows, attn_splits(p, path, rows));
  }
  if (op == DSA_OP_FORWARD) {
    const ForwardPlan f = plan_forward(p, path, true);
    return f.total();
  }
  if (op == DSA_OP_TOPK) {
    const int rows = p.batch * p.q_len;
    const int L = topk_sliced_len(rows, p.kv_len, p.topk);
    size_t hist_bytes;
    return L == 0 ? 0 : topk_sliced_bytes(rows, p.kv_len, L, &hist_bytes);
  }
  return 0;
}

int32_t dsa_forward_chunks(const dsa_problem_t* prob) {
  Path path;
  if (check_problem(prob, &path) != DSA_OK) return 0;
  return plan_forward(*prob, path, true).n_chunks;
}

dsa_status_t dsa_cache_append(const dsa_problem_t* prob, int32_t n_new,
                              const void* k_new, const uint8_t* k_new_scale, const void* kv_new,
                              void* k_idx, uint8_t* k_scale, void* kv, hipStream_t stream) {
  Path path;
  const dsa_status_t st = check_problem(prob, &path);
  if (st != DSA_OK) return st;
  const dsa_problem_t& p = *prob;
  if (n_new < 0 || p.kv_capacity == 0 || (int64_t)p.kv_len + n_new > p.kv_capacity) return DSA_ERR_INVALID_ARGUMENT;
  if (n_new == 0) return DSA_OK;
  const bool fp8 = path == kPathFP8;
  if (!k_new || !kv_new || !k_idx || !kv || (fp8 && (!k_new_scale || !k_scale))) return DSA_ERR_INVALID_ARGUMENT;
  const int kb = p.index_dim * (fp8 ? 1 : (p.index_dtype == DSA_F32 ? 4 : 2));
  const int vb = p.qk_dim * (p.attn_dtype == DSA_F32 ? 4 : 2);
  CacheAppend c;
  c.B = p.batch; c.n_new = n_new; c.pos = p.kv_len; c.cap = p.kv_capacity;
  c.k_new = k_new; c.ks_new = fp8 ? k_new_scale : nullptr; c.kv_new = kv_new;
  c.k = k_idx; c.ks = fp8 ? k_scale : nullptr; c.kv = kv;
  c.k_row_bytes = kb; c.kv_row_bytes = vb;
  return hip_status(launch_cache_append(c, stream));
}

dsa_status_t dsa_index_rotate_quantize(const void* x, dsa_dtype_t x_dtype, int64_t rows, int32_t dim,
                                       uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  if (rows < 0 || (x_dtype != DSA_BF16 && x_dtype != DSA_F32)) return DSA_ERR_INVALID_ARGUMENT;
  if (dim != 128) return DSA_ERR_UNSUPPORTED;
  if (rows == 0) return DSA_OK;
  if (!x || !codes || !scales || !aligned16(x) || (reinterpret_cast<uintptr_t>(codes) & 7u))
    return DSA_ERR_INVALID_ARGUMENT;
  return hip_status(launch_rotate_quant(x, x_dtype == DSA_F32, rows, codes, scales, stream));
}

dsa_status_t dsa_index_q_proj(const dsa_problem_t* prob, int32_t q_lora_rank, const void* cq, const void* wq_b,
                              void* q_idx, dsa_dtype_t q_dtype, hipStream_t stream) {
  Path path;
  const dsa_status_t st = check_problem(prob, &path);
  if (st != DSA_OK) return st;
  const dsa_problem_t& p = *prob;
  const int hd = p.index_heads * p.index_dim;
  return run_gemm(cq, wq_b, q_idx, p.batch * p.q_len, hd, q_lora_rank, 1, q_lora_rank, q_lora_rank, hd, 0, 0, 0,
                  q_dtype, stream);
}

dsa_status_t dsa_head_weights_proj(const dsa_problem_t* prob, int32_t dim, const void* x, const void* w_proj,
                                   float* head_w, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  Path path;
  const dsa_status_t st = check_problem(prob, &path);
  if (st != DSA_OK) return st;
  const dsa_problem_t& p = *prob;
  return run_gemm(x, w_proj, head_w, p.batch * p.q_len, p.index_heads, dim, 1, dim, dim, p.index_heads, 0, 0, 0,
                  DSA_F32, stream, workspace, workspace_bytes);
}

size_t dsa_head_weights_workspace_size(const dsa_problem_t* prob, int32_t dim) {
  Path path;
  if (check_problem(prob, &path) != DSA_OK || dim < 1) return 0;
  size_t need = 0;
  gemm_ksplit(prob->batch * prob->q_len, prob->index_heads, dim, 1, &need);
  return need;
}

dsa_status_t dsa_out_unabsorb(const dsa_problem_t* prob, int32_t v_head_dim, const void* o_latent, const void* w_uv,
                              void* out, dsa_dtype_t out_dtype, hipStream_t stream) {
  Path path;
  const dsa_status_t st = check_problem(prob, &path);
  if (st != DSA_OK) return st;
  const dsa_problem_t& p = *prob;
  if (v_head_dim < 1) return DSA_ERR_INVALID_ARGUMENT;
  const int NH = p.attn_heads, Dv = p.v_dim;
  // batch z = head: A rows are tokens with stride NH * Dv, offset z * Dv
  return run_gemm(o_latent, w_uv, out, p.batch * p.q_len, v_head_dim, Dv, NH, (int64_t)NH * Dv, Dv,
                  (int64_t)NH * v_head_dim, Dv, (int64_t)v_head_dim * Dv, v_head_dim, out_dtype, stream);
}

int32_t dsa_forward_attn_splits(const dsa_problem_t* prob) {
  Path path;
  if (check_problem(prob, &path) != DSA_OK) return 0;
  const ForwardPlan f = plan_forward(*prob, path, true);
  return attn_splits(*prob, path, prob->batch * f.chunk);
}

int32_t dsa_forward_topk_slice_len(const dsa_problem_t* prob) {
  Path path;
  if (check_problem(prob, &path) != DSA_OK) return 0;
  return plan_forward(*prob, path, true).tk_sl_len;
}

int32_t dsa_forward_topk_list_slots(const dsa_problem_t* prob) {
  Path path;
  if (check_problem(prob, &path) != DSA_OK) return 0;
  return plan_forward(*prob, path, true).tk_cand_m;
}

const char* dsa_status_string(dsa_status_t s) {
  switch (s) {
    case DSA_OK: return "ok";
    case DSA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case DSA_ERR_UNSUPPORTED: return "unsupported problem (dtype combination or dims)";
    case DSA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case DSA_ERR_HIP: return "HIP runtime or launch error";
    case DSA_ERR_EXCEEDS_SCRATCH: return "problem needs more than the library's static scratch (DSA_STATIC_SCRATCH_BYTES)";
  }
  return "unknown status";
}

int32_t dsa_abi_version(void) { return DSA_ABI_VERSION; }

}  // extern "C"
