// C ABI of the CSA hot path: argument validation, workspace layout and launch sequencing.
// Every check runs on the host before anything is enqueued; kernels never see an argument that
// could send them out of bounds (device-resident values are masked inside the kernels).
#include <cmath>
#include <cstdlib>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include <hip/hip_runtime.h>

#include "../../include/csa.h"
#include "csa_internal.h"

namespace {

thread_local int32_t g_last_hip = 0;

struct ProfRec {
  std::string name;
  hipEvent_t start, stop;
  bool used;   // attached to a launch
};
// Diagnostics only (csa_profile_*): the one piece of process-wide mutable state, guarded by a mutex
// so that calls from several host threads may record at once.
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<ProfRec> g_prof;

constexpr int kWin = 128;
constexpr int kHistBins = 4096;
constexpr int64_t kMaxEntries = (int64_t)1 << 30;
constexpr int32_t kMaxSlotsPerQuery = 16384;   // attention index-list length (window + compressed)
constexpr int32_t kMaxQueriesPerReq = 16;      // multi-query decode: tokens decoded together

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }
bool kv_fmt_ok(int f) { return f == CSA_KV_F32 || f == CSA_KV_BF16 || f == CSA_KV_FP8NOPE_BF16ROPE; }

csa_status hip_status(hipError_t e) {
  if (e == hipSuccess) return CSA_OK;
  g_last_hip = (int32_t)e;
  return CSA_ERR_HIP;
}

// ---- workspace carving ------------------------------------------------------------------------
struct Carver {
  uint8_t* base;
  size_t off = 0;
  explicit Carver(void* b) : base((uint8_t*)b) {}
  template <class T>
  T* take(size_t bytes) {
    T* p = base ? (T*)(base + off) : nullptr;
    off += align256(bytes);
    return p;
  }
};

struct TopkWs {
  uint32_t* hist;
  uint32_t* counters;
  int32_t* sel;
  uint2* cand;
};

TopkWs carve_topk(Carver& c, int32_t Q, int64_t max_n_vis, int32_t k) {
  TopkWs w;
  w.hist = c.take<uint32_t>((size_t)Q * kHistBins * 4);
  w.counters = c.take<uint32_t>((size_t)Q * 8 * 4);
  w.sel = c.take<int32_t>((size_t)Q * k * 4);
  w.cand = c.take<uint2>((size_t)Q * (size_t)(max_n_vis > 0 ? max_n_vis : 1) * 8);
  return w;
}

int64_t round64(int64_t x) { return (x + 63) / 64 * 64; }

struct PathWs {
  int32_t* n_vis;
  int32_t* q_req;
  int32_t* idx;
  float* logits;
  int64_t ld;
  TopkWs tk;
  float* part;
  int32_t* rows;     // [rows][k] compressed KV rows of the selection (one-block selections only)
  uint2* sk_top;     // long decode rows: per-wave sketches [rows][sk_waves][8] and bounds
  uint32_t* sk_bound;
  int64_t sk_waves;
};

// Which selection a fused call runs, from the visible-entry bound its workspace was sized for:
// one block per query over the whole row (short rows), one block per query over the indexer's
// per-wave sketches (long rows of a decode, one or several queries per request), or the multi-launch histogram
// selection (everything else).  The workspace layout depends on it, so a call and its workspace
// query decide it from the same numbers.
enum SelPath { kPathSingle, kPathSketch, kPathMulti };

SelPath sel_path(int mode, int32_t S, int64_t n, int32_t k) {
  if (csa::topk_single_ok(n, k)) return kPathSingle;
  if (mode == 1 && csa::topk_sketch_ok(n, k)) return kPathSketch;
  return kPathMulti;
}

PathWs carve_path(Carver& c, int32_t rows, int32_t H, int64_t max_n_vis, int32_t k, SelPath path) {
  PathWs w{};
  w.n_vis = c.take<int32_t>((size_t)rows * 4);
  w.q_req = c.take<int32_t>((size_t)rows * 4);
  w.idx = c.take<int32_t>((size_t)rows * (kWin + k) * 4);
  w.ld = round64(max_n_vis > 0 ? max_n_vis : 1);
  w.logits = c.take<float>((size_t)rows * (size_t)w.ld * 4);
  if (path == kPathMulti) w.tk = carve_topk(c, rows, max_n_vis, k);
  w.part = c.take<float>(csa::attn_partial_bytes(rows, H, kWin + k));
  if (path != kPathMulti) w.rows = c.take<int32_t>((size_t)rows * k * 4);
  if (path == kPathSketch) {
    w.sk_waves = csa::topk_sketch_waves(max_n_vis > 0 ? max_n_vis : 1);
    w.sk_top = c.take<uint2>((size_t)rows * (size_t)w.sk_waves * 8 * sizeof(uint2));
    w.sk_bound = c.take<uint32_t>((size_t)rows * (size_t)w.sk_waves * 4);
  }
  return w;
}

csa_status check_idx_struct(const csa_paged_idx* k, int32_t dt) {
  if (!k || !k->keys || !k->page_table) return CSA_ERR_NULL;
  if (k->dt != dt) return CSA_ERR_DTYPE;
  if ((dt == CSA_FP8_E4M3FN || dt == CSA_FP4_E2M1) && !k->scales) return CSA_ERR_NULL;
  if (dt == CSA_F32 && k->scales) return CSA_ERR_DTYPE;
  if (k->num_pages < 1 || k->max_pages < 1) return CSA_ERR_SHAPE;
  if (!aligned(k->keys, 16) || !aligned(k->page_table, 4) || (k->scales && !aligned(k->scales, 4))) return CSA_ERR_ALIGN;
  return CSA_OK;
}

csa_status check_kv_struct(const csa_paged_kv* c) {
  if (!c || !c->rows || !c->page_table) return CSA_ERR_NULL;
  if (!kv_fmt_ok(c->fmt)) return CSA_ERR_DTYPE;
  if (c->num_pages < 1 || c->max_pages < 1) return CSA_ERR_SHAPE;
  if (!aligned(c->rows, 16) || !aligned(c->page_table, 4)) return CSA_ERR_ALIGN;
  return CSA_OK;
}

csa_status check_indexer_inputs(const void* qI, const uint8_t* qI_scale, int32_t qI_dt, const float* w, int32_t HI) {
  if (!qI || !w) return CSA_ERR_NULL;
  if (qI_dt != CSA_F32 && qI_dt != CSA_FP8_E4M3FN && qI_dt != CSA_FP4_E2M1) return CSA_ERR_DTYPE;
  if (qI_dt != CSA_F32 && !qI_scale) return CSA_ERR_NULL;
  if (HI < 1 || HI > 64) return CSA_ERR_SHAPE;
  if (!aligned(qI, 16) || !aligned(w, 4)) return CSA_ERR_ALIGN;
  return CSA_OK;
}

csa_status check_attn_common(const void* q, int32_t q_dt, int32_t H, const float* sink, const void* out,
                             int32_t out_dt, float scale) {
  if (!q || !sink || !out) return CSA_ERR_NULL;
  if ((q_dt != CSA_F32 && q_dt != CSA_BF16) || (out_dt != CSA_F32 && out_dt != CSA_BF16)) return CSA_ERR_DTYPE;
  if (H < 1 || H > 128) return CSA_ERR_SHAPE;
  if (!std::isfinite(scale)) return CSA_ERR_SHAPE;
  if (!aligned(q, 16) || !aligned(out, 16) || !aligned(sink, 4)) return CSA_ERR_ALIGN;
  return CSA_OK;
}

// CSA_FAULT_INJECT=launch (read once per process): every entry point fails as a kernel launch
// would, with CSA_ERR_HIP and hipErrorLaunchFailure, after validating its arguments and before
// enqueuing anything.  For tests of callers' error handling; off by default.
bool fault_inject_launch() {
  static const bool on = [] {
    const char* e = getenv("CSA_FAULT_INJECT");
    return e != nullptr && strcmp(e, "launch") == 0;
  }();
  return on;
}

csa_status injected_fault() {
  if (!fault_inject_launch()) return CSA_OK;
  g_last_hip = (int32_t)hipErrorLaunchFailure;
  return CSA_ERR_HIP;
}

#define CSA_TRY(x)                      \
  do {                                  \
    csa_status _s = (x);                \
    if (_s != CSA_OK) return _s;        \
  } while (0)

#define CSA_HIP(x)                      \
  do {                                  \
    hipError_t _e = (x);                \
    if (_e != hipSuccess) return hip_status(_e); \
  } while (0)

}  // namespace

namespace csa {

ProfScope::ProfScope(const char* name, hipStream_t) : slot(-1) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (!g_prof_on) return;
  ProfRec r;
  r.name = name;
  r.used = false;
  if (hipEventCreate(&r.start) != hipSuccess) return;
  if (hipEventCreate(&r.stop) != hipSuccess) {
    (void)hipEventDestroy(r.start);
    return;
  }
  g_prof.push_back(r);
  slot = (int)g_prof.size() - 1;
  ev0 = r.start;
  ev1 = r.stop;
}

int32_t record_hip_error(hipError_t e) {
  g_last_hip = (int32_t)e;
  return CSA_ERR_HIP;
}

void ProfScope::mark() {
  if (slot < 0) return;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (slot < (int)g_prof.size()) g_prof[slot].used = true;
}

}  // namespace csa

extern "C" {

const char* csa_status_string(int32_t s) {
  switch (s) {
    case CSA_OK: return "ok";
    case CSA_ERR_NULL: return "required pointer is NULL";
    case CSA_ERR_SHAPE: return "size out of range";
    case CSA_ERR_DTYPE: return "unknown or unsupported dtype/format";
    case CSA_ERR_ALIGN: return "pointer not aligned";
    case CSA_ERR_WORKSPACE: return "workspace missing or too small";
    case CSA_ERR_UNSUPPORTED: return "unsupported combination";
    case CSA_ERR_HIP: return "HIP launch failed";
    case CSA_ERR_SCRATCH: return "the call needs more than the static scratch array holds";
    default: return "unknown status";
  }
}

int32_t csa_last_hip_error(void) { return g_last_hip; }

csa_status csa_debug_violations(uint64_t* count) {
  if (!count) return CSA_ERR_NULL;
#ifdef CSA_DEBUG_CHECKS
  const uint64_t parts[3] = {csa::debug_take_violations_attention(), csa::debug_take_violations_indexer(),
                             csa::debug_take_violations_topk()};
  uint64_t n = 0;
  for (uint64_t p : parts) {
    if (p == ~0ull) return (csa_status)csa::record_hip_error(hipErrorInvalidSymbol);
    n += p;
  }
  *count = n;
  return CSA_OK;
#else
  *count = 0;
  return CSA_ERR_UNSUPPORTED;
#endif
}

csa_status csa_profile_enable(int32_t on) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_on = on != 0;
  return CSA_OK;
}

csa_status csa_profile_reset(void) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (auto& r : g_prof) {
    if (r.used) (void)hipEventSynchronize(r.stop);
    (void)hipEventDestroy(r.start);
    (void)hipEventDestroy(r.stop);
  }
  g_prof.clear();
  return CSA_OK;
}

csa_status csa_profile_collect(const char* kernel, double* total_ms, int64_t* launches) {
  if (!kernel || !total_ms || !launches) return CSA_ERR_NULL;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  double tot = 0.0;
  int64_t n = 0;
  for (auto& r : g_prof) {
    if (r.name != kernel || !r.used) continue;
    hipError_t e = hipEventSynchronize(r.stop);
    if (e != hipSuccess) return hip_status(e);
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, r.start, r.stop);
    if (e != hipSuccess) return hip_status(e);
    tot += ms;
    ++n;
  }
  *total_ms = tot;
  *launches = n;
  return CSA_OK;
}

// ------------------------------------------------------------------------------------------------
csa_status csa_indexer_logits(const void* qI, const uint8_t* qI_scale, int32_t qI_dt, const float* w,
                              const csa_paged_idx* keys, const int32_t* q_req, int32_t n_req,
                              const int32_t* n_vis, int32_t Q, int32_t HI, int64_t max_n_vis,
                              float* logits, int64_t ld, hipStream_t stream) {
  CSA_TRY(check_indexer_inputs(qI, qI_scale, qI_dt, w, HI));
  CSA_TRY(check_idx_struct(keys, qI_dt));
  if (!q_req || !n_vis || !logits) return CSA_ERR_NULL;
  if (Q < 1 || Q > 65535 || n_req < 1) return CSA_ERR_SHAPE;
  if (max_n_vis < 0 || max_n_vis > kMaxEntries || ld < max_n_vis) return CSA_ERR_SHAPE;
  if (!aligned(q_req, 4) || !aligned(n_vis, 4) || !aligned(logits, 4)) return CSA_ERR_ALIGN;
  csa::IndexerArgs a{};
  a.qI = qI; a.qI_scale = qI_scale; a.dt = qI_dt; a.w = w;
  a.keys = keys->keys; a.kscale = keys->scales; a.num_pages = keys->num_pages;
  a.page_table = keys->page_table; a.max_pages = keys->max_pages;
  a.q_req = q_req; a.n_req = n_req; a.n_vis = n_vis; a.Q = Q; a.HI = HI;
  a.max_n_vis = max_n_vis; a.logits = logits; a.ld = ld; a.hist = nullptr;
  CSA_TRY(injected_fault());
  return hip_status(csa::launch_indexer(a, stream));
}

size_t csa_topk_workspace_bytes(int32_t Q, int64_t max_n_vis, int32_t k) {
  if (Q < 1 || k < 1 || max_n_vis < 0) return 0;
  Carver c(nullptr);
  carve_topk(c, Q, max_n_vis, k);
  return c.off;
}

csa_status csa_topk(const float* logits, int64_t ld, const int32_t* n_vis, int32_t Q, int64_t max_n_vis,
                    int32_t k, int32_t* idx, int64_t ld_idx, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!logits || !n_vis || !idx) return CSA_ERR_NULL;
  if (Q < 1 || Q > 65535 || k < 1 || k > 2048) return CSA_ERR_SHAPE;
  if (max_n_vis < 0 || max_n_vis > kMaxEntries || ld < max_n_vis || ld_idx < k) return CSA_ERR_SHAPE;
  if (!aligned(logits, 4) || !aligned(n_vis, 4) || !aligned(idx, 4)) return CSA_ERR_ALIGN;
  const size_t need = csa_topk_workspace_bytes(Q, max_n_vis, k);
  if (!ws || ws_bytes < need) return CSA_ERR_WORKSPACE;
  if (!aligned(ws, 16)) return CSA_ERR_ALIGN;
  CSA_TRY(injected_fault());
  Carver c(ws);
  TopkWs w = carve_topk(c, Q, max_n_vis, k);
  if (csa::topk_single_ok(max_n_vis, k) && ld % 4 == 0 && aligned(logits, 16)) {
    csa::TopkArgs t{};
    t.logits = logits; t.ld = ld; t.n_vis = n_vis; t.Q = Q; t.max_n_vis = max_n_vis; t.k = k;
    t.idx = idx; t.ld_idx = ld_idx; t.win_mode = 0;
    return hip_status(csa::launch_topk_single(t, stream));
  }
  csa::PrepArgs p{};
  p.zero_ptr = w.hist;
  p.zero_words = (int64_t)((uint8_t*)w.sel - (uint8_t*)w.hist) / 4;   // hist + counters
  p.mode = 0; p.ratio = 4;
  CSA_HIP(csa::launch_prep(p, stream));
  csa::TopkArgs t{};
  t.logits = logits; t.ld = ld; t.n_vis = n_vis; t.Q = Q; t.max_n_vis = max_n_vis; t.k = k;
  t.idx = idx; t.ld_idx = ld_idx; t.hist = w.hist; t.counters = w.counters; t.sel = w.sel;
  t.cand = w.cand; t.cand_cap = max_n_vis > 0 ? max_n_vis : 1;
  CSA_HIP(csa::launch_topk_hist(t, stream));
  return hip_status(csa::launch_topk_select(t, stream));
}

size_t csa_sparse_attn_workspace_bytes(int32_t Q, int32_t H, int32_t n_idx) {
  if (Q < 1 || H < 1 || n_idx < 1) return 0;
  return csa::attn_partial_bytes(Q, H, n_idx);
}

csa_status csa_sparse_attn(const void* q, int32_t q_dt, int32_t Q, int32_t H, const float* sink,
                           const void* win_rows, int32_t win_fmt, int64_t win_rows_per_req,
                           const csa_paged_kv* comp, const int32_t* q_req, int32_t n_req, const int32_t* idx,
                           int64_t ld_idx, int32_t n_win, int32_t n_comp, float softmax_scale, void* out,
                           int32_t out_dt, void* ws, size_t ws_bytes, hipStream_t stream) {
  CSA_TRY(check_attn_common(q, q_dt, H, sink, out, out_dt, softmax_scale));
  if (!q_req || !idx) return CSA_ERR_NULL;
  if (Q < 1 || Q > 65535 || n_req < 1 || n_win < 0 || n_comp < 0) return CSA_ERR_SHAPE;
  const int32_t n_idx = n_win + n_comp;
  if (n_idx < 1 || n_idx > kMaxSlotsPerQuery || ld_idx < n_idx) return CSA_ERR_SHAPE;
  if (n_win > 0) {
    if (!win_rows) return CSA_ERR_NULL;
    if (!kv_fmt_ok(win_fmt)) return CSA_ERR_DTYPE;
    if (win_rows_per_req < 0 || win_rows_per_req > kMaxEntries) return CSA_ERR_SHAPE;
    if (!aligned(win_rows, 16)) return CSA_ERR_ALIGN;
  }
  if (n_comp > 0) CSA_TRY(check_kv_struct(comp));
  if (!aligned(q_req, 4) || !aligned(idx, 4)) return CSA_ERR_ALIGN;
  const size_t need = csa_sparse_attn_workspace_bytes(Q, H, n_idx);
  if (need > 0 && (!ws || ws_bytes < need)) return CSA_ERR_WORKSPACE;
  if (need > 0 && !aligned(ws, 16)) return CSA_ERR_ALIGN;
  csa::AttnArgs a{};
  a.q = q; a.q_dt = q_dt; a.Q = Q; a.H = H; a.sink = sink;
  a.win = n_win > 0 ? (const uint8_t*)win_rows : nullptr; a.win_fmt = n_win > 0 ? win_fmt : 0;
  a.win_rows_per_req = win_rows_per_req;
  if (n_comp > 0) {
    a.comp = (const uint8_t*)comp->rows; a.comp_fmt = comp->fmt; a.comp_num_pages = comp->num_pages;
    a.page_table = comp->page_table; a.max_pages = comp->max_pages;
  }
  a.q_req = q_req; a.n_req = n_req; a.idx = idx; a.ld_idx = ld_idx; a.n_win = n_win; a.n_comp = n_comp;
  a.softmax_scale = softmax_scale; a.out = out; a.out_dt = out_dt;
  a.n_split = csa::attn_uses_matrix_cores(q_dt, a.win_fmt, a.comp_fmt, n_win, n_comp)
                  ? csa::plan_attn_split(Q, H, n_idx, q_dt) : 1;
  a.part = (float*)ws;
  CSA_TRY(injected_fault());
  return hip_status(csa::launch_attention(a, stream));
}

// ------------------------------------------------------------------------------------------------
static csa_status run_path(int mode, int32_t rows, int32_t H, int32_t HI, int32_t k, const void* q, int32_t q_dt,
                           const float* sink, const void* qI, const uint8_t* qI_scale, int32_t qI_dt,
                           const float* w, const csa_paged_idx* keys, const csa_paged_kv* comp,
                           const void* win, int32_t win_fmt, int64_t win_rows_per_req, const int32_t* ctx_len,
                           int64_t max_ctx, int64_t pos0, int64_t max_n_vis, float softmax_scale, void* out,
                           int32_t out_dt, int32_t* idx_out, void* ws, size_t ws_bytes, int64_t n_query,
                           hipStream_t stream, int32_t S = 1, int32_t ring = kWin) {
  // the workspace is laid out for n_query visible entries (what the workspace query was given);
  // the kernels see the call's own bound max_n_vis <= n_query
  const SelPath path = sel_path(mode, S, n_query, k);
  Carver sizer(nullptr);
  carve_path(sizer, rows, H, n_query, k, path);
  if (!ws || ws_bytes < sizer.off) return CSA_ERR_WORKSPACE;
  if (!aligned(ws, 16)) return CSA_ERR_ALIGN;
  if (idx_out && !aligned(idx_out, 4)) return CSA_ERR_ALIGN;
  CSA_TRY(injected_fault());
  Carver c(ws);
  PathWs pw = carve_path(c, rows, H, n_query, k, path);
  int32_t* idx = idx_out ? idx_out : pw.idx;
  const int64_t ld_idx = kWin + k;
  // Short rows: the indexer and a one-block-per-query selection derive visibility from ctx_len /
  // pos0 themselves, so no preparation launch and no zeroed histogram are needed.  Long decode
  // rows likewise: the indexer leaves per-wave sketches and one block per
  // query selects from them.
  const bool single = path == kPathSingle;
  const bool sketch = path == kPathSketch;
  const bool one_block = single || sketch;

  if (!one_block) {
    csa::PrepArgs p{};
    p.zero_ptr = pw.tk.hist;
    p.zero_words = (int64_t)((uint8_t*)pw.tk.sel - (uint8_t*)pw.tk.hist) / 4;
    p.mode = mode; p.rows = rows; p.ctx_len = ctx_len; p.max_ctx = max_ctx; p.pos0 = pos0;
    p.idx = idx; p.ld_idx = ld_idx; p.n_vis_out = pw.n_vis; p.q_req_out = pw.q_req;
    p.ratio = 4; p.q_per_req = S; p.ring = ring;
    CSA_HIP(csa::launch_prep(p, stream));
  }

  csa::IndexerArgs ia{};
  ia.qI = qI; ia.qI_scale = qI_scale; ia.dt = qI_dt; ia.w = w;
  ia.keys = keys->keys; ia.kscale = keys->scales; ia.num_pages = keys->num_pages;
  ia.page_table = keys->page_table; ia.max_pages = keys->max_pages;
  ia.q_req = pw.q_req; ia.n_req = mode == 1 ? rows / S : 1; ia.n_vis = pw.n_vis; ia.Q = rows; ia.HI = HI;
  ia.max_n_vis = max_n_vis; ia.logits = pw.logits; ia.ld = pw.ld; ia.hist = one_block ? nullptr : pw.tk.hist;
  ia.vis_mode = one_block ? mode : 0; ia.ctx_len = ctx_len; ia.max_ctx = max_ctx; ia.pos0 = pos0; ia.q_per_req = S;
  ia.visible_only = true;
  if (sketch) {
    ia.sk_top = pw.sk_top; ia.sk_bound = pw.sk_bound; ia.sk_waves = pw.sk_waves;
    // rows of at least 64k entries hold k real sketch entries (8 per 512-entry span): they store
    // no scores, and the selection rescores one when its sketches cannot decide it
    ia.sk_rescore_from = csa::sketch_rescore_from(k);
  }
  CSA_HIP(csa::launch_indexer(ia, stream));

  csa::TopkArgs t{};
  t.logits = pw.logits; t.ld = pw.ld; t.n_vis = pw.n_vis; t.Q = rows; t.max_n_vis = max_n_vis; t.k = k;
  t.idx = idx + kWin; t.ld_idx = ld_idx; t.hist = pw.tk.hist; t.counters = pw.tk.counters; t.sel = pw.tk.sel;
  t.cand = pw.tk.cand; t.cand_cap = max_n_vis > 0 ? max_n_vis : 1;
  t.win_mode = one_block ? mode : 0; t.ctx_len = ctx_len; t.max_ctx = max_ctx; t.pos0 = pos0;
  t.q_per_req = S; t.ring = ring;
  if (one_block) {
    // the selection also resolves its rows through the page table, which it loads while the
    // scores load, so the attention prologue saves one dependent round trip
    t.rows = pw.rows; t.ld_rows = k; t.page_table = comp->page_table; t.max_pages = comp->max_pages;
    t.num_pages = comp->num_pages;
  }
  if (sketch) { t.sk_top = pw.sk_top; t.sk_bound = pw.sk_bound; t.sk_waves = pw.sk_waves; t.ia = ia; }
  // one query per request with one-block or sketch rows: the attention launch runs the selection
  // (inside its own blocks when it can, else as its own launch first)
  const bool sel_in_attn = (single || sketch) && mode == 1 && S == 1;
  if (!sel_in_attn)
    CSA_HIP(single ? csa::launch_topk_single(t, stream)
                   : (sketch ? csa::launch_topk_sketch(t, stream) : csa::launch_topk_select(t, stream)));

  csa::AttnArgs a{};
  a.q = q; a.q_dt = q_dt; a.Q = rows; a.H = H; a.sink = sink;
  a.win = (const uint8_t*)win; a.win_fmt = win_fmt; a.win_rows_per_req = win_rows_per_req;
  a.comp = (const uint8_t*)comp->rows; a.comp_fmt = comp->fmt; a.comp_num_pages = comp->num_pages;
  a.page_table = comp->page_table; a.max_pages = comp->max_pages;
  a.q_req = pw.q_req; a.n_req = mode == 1 ? rows / S : 1; a.idx = idx; a.ld_idx = ld_idx; a.n_win = kWin; a.n_comp = k;
  a.softmax_scale = softmax_scale; a.out = out; a.out_dt = out_dt;
  a.n_split = csa::attn_uses_matrix_cores(q_dt, win_fmt, comp->fmt, kWin, k) ? csa::plan_attn_split(rows, H, kWin + k, q_dt) : 1;
  a.part = pw.part;
  a.req_mode = mode;
  a.q_per_req = S;
  if (mode == 2) { a.trim_ratio = 4; a.pos0 = pos0; }   // selection pads past min(n_vis, k) with -1
  a.stream_rows = mode == 1 && S == 1;   // one query per request: each row is gathered once
  if (one_block) { a.rows = pw.rows; a.ld_rows = k; }
  if (sel_in_attn) a.sel = &t;
  return hip_status(csa::launch_attention(a, stream));
}

static csa_status check_path(int32_t rows, int32_t H, int32_t HI, int32_t k, const void* q, int32_t q_dt,
                             const float* sink, const void* qI, const uint8_t* qI_scale, int32_t qI_dt,
                             const float* w, const csa_paged_idx* keys, const csa_paged_kv* comp, const void* win,
                             int32_t win_fmt, float scale, void* out, int32_t out_dt) {
  CSA_TRY(check_attn_common(q, q_dt, H, sink, out, out_dt, scale));
  CSA_TRY(check_indexer_inputs(qI, qI_scale, qI_dt, w, HI));
  CSA_TRY(check_idx_struct(keys, qI_dt));
  CSA_TRY(check_kv_struct(comp));
  if (!win) return CSA_ERR_NULL;
  if (!kv_fmt_ok(win_fmt)) return CSA_ERR_DTYPE;
  if (!aligned(win, 16)) return CSA_ERR_ALIGN;
  if (rows < 1 || rows > 65535 || k < 1 || k > 2048) return CSA_ERR_SHAPE;
  if (comp->max_pages != keys->max_pages) return CSA_ERR_SHAPE;
  return CSA_OK;
}

size_t csa_decode_workspace_bytes(int32_t B, int32_t H, int32_t HI, int64_t max_ctx, int32_t k) {
  if (B < 1 || H < 1 || HI < 1 || k < 1 || max_ctx < 0) return 0;
  Carver c(nullptr);
  carve_path(c, B, H, max_ctx / 4, k, sel_path(1, 1, max_ctx / 4, k));
  return c.off;
}

csa_status csa_decode(int32_t B, int32_t H, int32_t HI, int32_t k, const void* q, int32_t q_dt, const float* sink,
                      const void* qI, const uint8_t* qI_scale, int32_t qI_dt, const float* w,
                      const csa_paged_idx* keys, const csa_paged_kv* comp, const void* win_ring, int32_t win_fmt,
                      const int32_t* ctx_len, int64_t max_ctx, float softmax_scale, void* out, int32_t out_dt,
                      int32_t* idx_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  CSA_TRY(check_path(B, H, HI, k, q, q_dt, sink, qI, qI_scale, qI_dt, w, keys, comp, win_ring, win_fmt,
                     softmax_scale, out, out_dt));
  if (!ctx_len) return CSA_ERR_NULL;
  if (!aligned(ctx_len, 4)) return CSA_ERR_ALIGN;
  if (max_ctx < 0 || max_ctx > INT32_MAX) return CSA_ERR_SHAPE;
  const int64_t max_n_vis = std::min<int64_t>(max_ctx / 4, (int64_t)keys->max_pages * 64);
  return run_path(1, B, H, HI, k, q, q_dt, sink, qI, qI_scale, qI_dt, w, keys, comp, win_ring, win_fmt, kWin,
                  ctx_len, max_ctx, 0, max_n_vis, softmax_scale, out, out_dt, idx_out, ws, ws_bytes, max_ctx / 4, stream);
}

size_t csa_decode_multi_workspace_bytes(int32_t B, int32_t S, int32_t H, int32_t HI, int64_t max_ctx, int32_t k) {
  if (B < 1 || S < 1 || S > kMaxQueriesPerReq || H < 1 || HI < 1 || k < 1 || max_ctx < 0) return 0;
  Carver c(nullptr);
  carve_path(c, B * S, H, max_ctx / 4, k, sel_path(1, S, max_ctx / 4, k));
  return c.off;
}

csa_status csa_decode_multi(int32_t B, int32_t S, int32_t H, int32_t HI, int32_t k, const void* q, int32_t q_dt,
                            const float* sink, const void* qI, const uint8_t* qI_scale, int32_t qI_dt, const float* w,
                            const csa_paged_idx* keys, const csa_paged_kv* comp, const void* win_ring,
                            int32_t win_fmt, int32_t ring_slots, const int32_t* ctx_len, int64_t max_ctx,
                            float softmax_scale, void* out, int32_t out_dt, int32_t* idx_out, void* ws,
                            size_t ws_bytes, hipStream_t stream) {
  if (S < 1 || S > kMaxQueriesPerReq || B < 1 || (int64_t)B * S > 65535) return CSA_ERR_SHAPE;
  CSA_TRY(check_path(B * S, H, HI, k, q, q_dt, sink, qI, qI_scale, qI_dt, w, keys, comp, win_ring, win_fmt,
                     softmax_scale, out, out_dt));
  if (!ctx_len) return CSA_ERR_NULL;
  if (!aligned(ctx_len, 4)) return CSA_ERR_ALIGN;
  if (max_ctx < 0 || max_ctx > INT32_MAX) return CSA_ERR_SHAPE;
  if (ring_slots < kWin + S - 1 || ring_slots > (1 << 20)) return CSA_ERR_SHAPE;
  const int64_t max_n_vis = std::min<int64_t>(max_ctx / 4, (int64_t)keys->max_pages * 64);
  return run_path(1, B * S, H, HI, k, q, q_dt, sink, qI, qI_scale, qI_dt, w, keys, comp, win_ring, win_fmt,
                  ring_slots, ctx_len, max_ctx, 0, max_n_vis, softmax_scale, out, out_dt, idx_out, ws, ws_bytes,
                  max_ctx / 4, stream, S, ring_slots);
}

size_t csa_prefill_workspace_bytes(int32_t Q, int32_t H, int32_t HI, int64_t T, int32_t k) {
  if (Q < 1 || H < 1 || HI < 1 || k < 1 || T < 0) return 0;
  Carver c(nullptr);
  carve_path(c, Q, H, T / 4, k, sel_path(2, 1, T / 4, k));
  return c.off;
}

csa_status csa_prefill(int32_t Q, int32_t H, int32_t HI, int32_t k, const void* q, int32_t q_dt, const float* sink,
                       const void* qI, const uint8_t* qI_scale, int32_t qI_dt, const float* w,
                       const csa_paged_idx* keys, const csa_paged_kv* comp, const void* raw_rows, int32_t raw_fmt,
                       int64_t T, int64_t pos0, float softmax_scale, void* out, int32_t out_dt, int32_t* idx_out,
                       void* ws, size_t ws_bytes, hipStream_t stream) {
  CSA_TRY(check_path(Q, H, HI, k, q, q_dt, sink, qI, qI_scale, qI_dt, w, keys, comp, raw_rows, raw_fmt,
                     softmax_scale, out, out_dt));
  if (T < 1 || T > INT32_MAX || pos0 < 0 || pos0 + Q > T) return CSA_ERR_SHAPE;
  const int64_t max_n_vis = std::min<int64_t>((pos0 + Q) / 4, (int64_t)keys->max_pages * 64);
  return run_path(2, Q, H, HI, k, q, q_dt, sink, qI, qI_scale, qI_dt, w, keys, comp, raw_rows, raw_fmt, T,
                  nullptr, 0, pos0, max_n_vis, softmax_scale, out, out_dt, idx_out, ws, ws_bytes, T / 4, stream);
}

}  // extern "C"

// ---- layers without an indexer ([P1] section 2.8 get_compress_topk_idxs, and the attention
// forward's "no indexer" branch): every visible compressed entry is attended, plus the window.
namespace {

struct HcaWs {
  int32_t* n_vis;
  int32_t* q_req;
  int32_t* idx;
  float* part;
};

HcaWs carve_hca(Carver& c, int32_t rows, int32_t H, int64_t n_comp) {
  HcaWs w;
  w.n_vis = c.take<int32_t>((size_t)rows * 4);
  w.q_req = c.take<int32_t>((size_t)rows * 4);
  w.idx = c.take<int32_t>((size_t)rows * (size_t)(kWin + n_comp) * 4);
  w.part = c.take<float>(csa::attn_partial_bytes(rows, H, (int)(kWin + n_comp)));
  return w;
}

csa_status run_hca(int mode, int32_t rows, int32_t H, const void* q, int32_t q_dt, const float* sink,
                   const csa_paged_kv* comp, const void* win, int32_t win_fmt, int64_t win_rows_per_req,
                   const int32_t* ctx_len, int64_t max_ctx, int64_t pos0, int32_t ratio, int64_t n_comp,
                   float softmax_scale, void* out, int32_t out_dt, void* ws, size_t ws_bytes, hipStream_t stream) {
  Carver c(ws);
  HcaWs w = carve_hca(c, rows, H, n_comp);
  if (!ws || ws_bytes < c.off) return CSA_ERR_WORKSPACE;
  if (!aligned(ws, 16)) return CSA_ERR_ALIGN;
  CSA_TRY(injected_fault());
  const int64_t ld_idx = kWin + n_comp;
  csa::PrepArgs p{};
  p.mode = mode; p.rows = rows; p.ctx_len = ctx_len; p.max_ctx = max_ctx; p.pos0 = pos0;
  p.idx = w.idx; p.ld_idx = ld_idx; p.n_vis_out = w.n_vis; p.q_req_out = w.q_req;
  p.ratio = ratio; p.comp_cols = n_comp;
  CSA_HIP(csa::launch_prep(p, stream));

  csa::AttnArgs a{};
  a.q = q; a.q_dt = q_dt; a.Q = rows; a.H = H; a.sink = sink;
  a.win = (const uint8_t*)win; a.win_fmt = win_fmt; a.win_rows_per_req = win_rows_per_req;
  const int nc = (int)n_comp;
  if (nc > 0) {
    a.comp = (const uint8_t*)comp->rows; a.comp_fmt = comp->fmt; a.comp_num_pages = comp->num_pages;
    a.page_table = comp->page_table; a.max_pages = comp->max_pages;
  }
  a.q_req = w.q_req; a.n_req = mode == 1 ? rows : 1; a.idx = w.idx; a.ld_idx = ld_idx; a.n_win = kWin;
  a.n_comp = nc; a.softmax_scale = softmax_scale; a.out = out; a.out_dt = out_dt;
  a.n_split = csa::attn_uses_matrix_cores(q_dt, win_fmt, a.comp_fmt, kWin, nc)
                  ? csa::plan_attn_split(rows, H, kWin + nc, q_dt) : 1;
  a.part = w.part;
  a.req_mode = mode;
  if (mode == 2) { a.trim_ratio = ratio; a.pos0 = pos0; }   // dense lists stop at the visible count
  a.stream_rows = mode == 1;   // decode: each request's rows belong to its one query
  return hip_status(csa::launch_attention(a, stream));
}

csa_status check_hca(int32_t rows, int32_t H, const void* q, int32_t q_dt, const float* sink,
                     const csa_paged_kv* comp, const void* win, int32_t win_fmt, int32_t ratio, float scale,
                     void* out, int32_t out_dt) {
  CSA_TRY(check_attn_common(q, q_dt, H, sink, out, out_dt, scale));
  CSA_TRY(check_kv_struct(comp));
  if (!win) return CSA_ERR_NULL;
  if (!kv_fmt_ok(win_fmt)) return CSA_ERR_DTYPE;
  if (!aligned(win, 16)) return CSA_ERR_ALIGN;
  if (rows < 1 || rows > 65535 || ratio < 1) return CSA_ERR_SHAPE;
  return CSA_OK;
}

int64_t hca_cols(int64_t n_vis_max, const csa_paged_kv* comp) {
  return std::min<int64_t>(n_vis_max, (int64_t)comp->max_pages * 64);
}

}  // namespace

extern "C" {

// ---- compressor ([P1] section 2.9): writes compressed entries into the caches
namespace {
csa_status compress_common(const void* kv_proj, const void* score_proj, int32_t proj_dt, int64_t ld_proj,
                           int64_t tok0, int64_t n_tok, int32_t ratio, int32_t D, const float* ape,
                           const float* norm_w, float eps, const float* rope_cos, const float* rope_sin,
                           int64_t c_begin, int32_t c_count, int32_t num_pages, const int32_t* page_table_row,
                           int32_t max_pages, csa::CompressArgs& a) {
  if (!kv_proj || !score_proj || !ape || !norm_w || !rope_cos || !rope_sin || !page_table_row) return CSA_ERR_NULL;
  if (proj_dt != CSA_F32 && proj_dt != CSA_BF16) return CSA_ERR_DTYPE;
  if (ratio != 4 && ratio != 128) return CSA_ERR_SHAPE;
  const int coff = ratio == 4 ? 2 : 1;
  if (ld_proj < (int64_t)coff * D || ld_proj % 8 != 0 || !std::isfinite(eps) || eps < 0.f) return CSA_ERR_SHAPE;
  if (c_begin < 0 || c_count < 0 || n_tok < 0 || tok0 < 0 || num_pages < 1 || max_pages < 1) return CSA_ERR_SHAPE;
  if (c_begin + c_count > (int64_t)max_pages * 64) return CSA_ERR_SHAPE;
  if (c_count > 0) {
    // every token the entries pool must have a projection row
    const int64_t first = (ratio == 4 && c_begin > 0) ? (c_begin - 1) * ratio : c_begin * ratio;
    if (first < tok0 || (c_begin + c_count) * ratio > tok0 + n_tok) return CSA_ERR_SHAPE;
  }
  if (!aligned(kv_proj, 16) || !aligned(score_proj, 16) || !aligned(ape, 16) || !aligned(norm_w, 16) ||
      !aligned(rope_cos, 16) || !aligned(rope_sin, 16) || !aligned(page_table_row, 4))
    return CSA_ERR_ALIGN;
  a.kv = kv_proj; a.score = score_proj; a.proj_dt = proj_dt == CSA_BF16 ? 1 : 0; a.ld = ld_proj; a.tok0 = tok0;
  a.ratio = ratio; a.D = D; a.ape = ape; a.norm_w = norm_w; a.eps = eps; a.rope_cos = rope_cos;
  a.rope_sin = rope_sin; a.c_begin = c_begin; a.c_count = c_count; a.num_pages = num_pages;
  a.page_table = page_table_row;
  return CSA_OK;
}
}  // namespace

csa_status csa_compress_kv(const void* kv_proj, const void* score_proj, int32_t proj_dt, int64_t ld_proj,
                           int64_t tok0, int64_t n_tok, int32_t ratio, const float* ape, const float* norm_w,
                           float eps, const float* rope_cos, const float* rope_sin, int64_t c_begin,
                           int32_t c_count, void* pool_rows, int32_t pool_fmt, int32_t num_pages,
                           const int32_t* page_table_row, int32_t max_pages, hipStream_t stream) {
  csa::CompressArgs a{};
  CSA_TRY(compress_common(kv_proj, score_proj, proj_dt, ld_proj, tok0, n_tok, ratio, 512, ape, norm_w, eps, rope_cos,
                          rope_sin, c_begin, c_count, num_pages, page_table_row, max_pages, a));
  if (!pool_rows) return CSA_ERR_NULL;
  if (!kv_fmt_ok(pool_fmt)) return CSA_ERR_DTYPE;
  if (!aligned(pool_rows, 16)) return CSA_ERR_ALIGN;
  a.out = (uint8_t*)pool_rows; a.out_fmt = pool_fmt;
  CSA_TRY(injected_fault());
  return hip_status(csa::launch_compress(a, stream));
}

csa_status csa_compress_index_keys(const void* kv_proj, const void* score_proj, int32_t proj_dt, int64_t ld_proj,
                                   int64_t tok0, int64_t n_tok, int32_t ratio, const float* ape,
                                   const float* norm_w, float eps, const float* rope_cos, const float* rope_sin,
                                   int64_t c_begin, int32_t c_count, void* keys, uint8_t* scales, int32_t key_dt,
                                   int32_t num_pages, const int32_t* page_table_row, int32_t max_pages,
                                   hipStream_t stream) {
  csa::CompressArgs a{};
  CSA_TRY(compress_common(kv_proj, score_proj, proj_dt, ld_proj, tok0, n_tok, ratio, 128, ape, norm_w, eps, rope_cos,
                          rope_sin, c_begin, c_count, num_pages, page_table_row, max_pages, a));
  if (!keys || !scales) return CSA_ERR_NULL;
  if (key_dt != CSA_FP8_E4M3FN && key_dt != CSA_FP4_E2M1) return CSA_ERR_DTYPE;
  if (!aligned(keys, 16)) return CSA_ERR_ALIGN;
  a.out = (uint8_t*)keys; a.out_fmt = key_dt; a.out_scales = scales;
  CSA_TRY(injected_fault());
  return hip_status(csa::launch_compress(a, stream));
}

size_t csa_hca_decode_workspace_bytes(int32_t B, int32_t H, int64_t max_ctx, int32_t ratio) {
  if (B < 1 || H < 1 || max_ctx < 0 || ratio < 1 || max_ctx / ratio + kWin > kMaxSlotsPerQuery) return 0;
  Carver c(nullptr);
  carve_hca(c, B, H, max_ctx / ratio);
  return c.off;
}

csa_status csa_hca_decode(int32_t B, int32_t H, const void* q, int32_t q_dt, const float* sink,
                          const csa_paged_kv* comp, const void* win_ring, int32_t win_fmt, const int32_t* ctx_len,
                          int64_t max_ctx, int32_t ratio, float softmax_scale, void* out, int32_t out_dt, void* ws,
                          size_t ws_bytes, hipStream_t stream) {
  CSA_TRY(check_hca(B, H, q, q_dt, sink, comp, win_ring, win_fmt, ratio, softmax_scale, out, out_dt));
  if (!ctx_len) return CSA_ERR_NULL;
  if (!aligned(ctx_len, 4)) return CSA_ERR_ALIGN;
  if (max_ctx < 0 || max_ctx > INT32_MAX) return CSA_ERR_SHAPE;
  const int64_t n_comp = hca_cols(max_ctx / ratio, comp);
  if (kWin + n_comp > kMaxSlotsPerQuery) return CSA_ERR_SHAPE;
  return run_hca(1, B, H, q, q_dt, sink, comp, win_ring, win_fmt, kWin, ctx_len, max_ctx, 0, ratio, n_comp,
                 softmax_scale, out, out_dt, ws, ws_bytes, stream);
}

size_t csa_hca_prefill_workspace_bytes(int32_t Q, int32_t H, int64_t T, int32_t ratio) {
  if (Q < 1 || H < 1 || T < 0 || ratio < 1 || T / ratio + kWin > kMaxSlotsPerQuery) return 0;
  Carver c(nullptr);
  carve_hca(c, Q, H, T / ratio);
  return c.off;
}

csa_status csa_hca_prefill(int32_t Q, int32_t H, const void* q, int32_t q_dt, const float* sink,
                           const csa_paged_kv* comp, const void* raw_rows, int32_t raw_fmt, int64_t T, int64_t pos0,
                           int32_t ratio, float softmax_scale, void* out, int32_t out_dt, void* ws, size_t ws_bytes,
                           hipStream_t stream) {
  CSA_TRY(check_hca(Q, H, q, q_dt, sink, comp, raw_rows, raw_fmt, ratio, softmax_scale, out, out_dt));
  if (T < 1 || T > INT32_MAX || pos0 < 0 || pos0 + Q > T) return CSA_ERR_SHAPE;
  const int64_t n_comp = hca_cols((pos0 + Q) / ratio, comp);
  if (kWin + n_comp > kMaxSlotsPerQuery) return CSA_ERR_SHAPE;
  return run_hca(2, Q, H, q, q_dt, sink, comp, raw_rows, raw_fmt, T, nullptr, 0, pos0, ratio, n_comp,
                 softmax_scale, out, out_dt, ws, ws_bytes, stream);
}

}  // extern "C"
