// Internal host-side interface between the C ABI layer (api.cpp) and the kernel launchers.
#pragma once
#include <hip/hip_runtime_api.h>
#include <hip/hip_vector_types.h>
#include <stdint.h>

namespace csa {

// Sizes and codes the kernels and the host planners (plan.cpp) share.
enum RowFmt : int { kRowF32 = 0, kRowBF16 = 1, kRowFP8 = 2 };   // KV row formats (CSA_KV_* codes)
constexpr int kSketchTop = 8;            // long-row sketch: largest scores kept per indexer wave
constexpr int kSketchSpan = 512;         // entries scored by one indexer wave (8 pages)
constexpr int kTile = 32;                // attention: slots per tile
constexpr int kMaxSlots = 1024;          // attention: slots of one block; longer lists are split
constexpr int kMaxSplit = 32;            // attention: key-range splits of one query
constexpr int kSingleMax = 1024 * 32;    // one-block selection: longest row (1024 threads of 32)
constexpr int kSingleMaxK = 2048;        // one-block selection: largest k
constexpr int kSketchMaxWaves = 2048;    // sketch selection: rows up to 2^20 entries
constexpr int kRowD = 512;               // head dim

// Debug builds only (-DCSA_DEBUG_CHECKS): masked-value counters of each kernel file, read and cleared.
uint64_t debug_take_violations_attention();
uint64_t debug_take_violations_indexer();
uint64_t debug_take_violations_topk();

// Records e as the calling thread's last HIP error and returns CSA_ERR_HIP.
int32_t record_hip_error(hipError_t e);

// Per-launch timing while profiling is on (see csa_profile_enable): the scope owns two events that
// CSA_LAUNCH (csa_device.h) attaches to the kernel's own dispatch, so they bracket its execution on the GPU, not
// its enqueue.  With profiling off both events are null and the launch is an ordinary one.
struct ProfScope {
  ProfScope(const char* name, hipStream_t s);
  void mark();   // the scope's events were attached to a launch
  int slot;
  hipEvent_t ev0 = nullptr, ev1 = nullptr;
};


struct IndexerArgs {
  const void* qI;             // [Q][HI][128] fp8 bytes or fp32
  const uint8_t* qI_scale;    // [Q][HI][4] E8M0 (fp8 only)
  int dt;                     // 0 = f32, 2 = fp8 e4m3fn, 3 = fp4 e2m1 (two per byte)
  const float* w;             // [Q][HI]
  const void* keys;           // [P][64][128]
  const uint8_t* kscale;      // [P][4][64]
  int num_pages;
  const int32_t* page_table;  // [n_req][max_pages]
  int max_pages;
  const int32_t* q_req;       // [Q]
  int n_req;
  const int32_t* n_vis;       // [Q]
  int Q, HI;
  int64_t max_n_vis;
  float* logits;              // [Q][ld]
  int64_t ld;
  uint32_t* hist;             // optional [Q][4096] coarse histogram of the written scores
  // 0: q_req / n_vis arrays; 1: decode (request q, n_vis = clamp(ctx_len[q], 0, max_ctx)/4);
  // 2: causal prefill of request 0 (n_vis = (pos0 + q + 1)/4)
  int vis_mode;
  const int32_t* ctx_len;
  int64_t max_ctx;
  int64_t pos0;
  int q_per_req = 1;          // decode: queries per request (query q belongs to request q / q_per_req)
  // true inside the fused paths: only columns c < n_vis of each row are written (the selection
  // reads nothing else); false for csa_indexer_logits, which also fills [n_vis, max_n_vis) with -inf
  bool visible_only = false;
  // optional (decode, one query per request, visible_only): per-wave sketch of each row for the
  // one-launch long-row selection: [Q][sk_waves][8] (order key, entry) and [Q][sk_waves] bounds
  uint2* sk_top = nullptr;
  uint32_t* sk_bound = nullptr;
  int64_t sk_waves = 0;
  // sketch rows with at least this many visible entries (> 0) store no scores: their sketches hold
  // at least k real entries, and the selection rescores such a row when the sketches cannot
  // decide it (rescore_span).  0: every row stores its scores.
  int64_t sk_rescore_from = 0;
};
hipError_t launch_indexer(const IndexerArgs& a, hipStream_t s);

struct TopkArgs {
  const float* logits;
  int64_t ld;
  const int32_t* n_vis;
  int Q;
  int64_t max_n_vis;
  int k;
  int32_t* idx;
  int64_t ld_idx;
  uint32_t* hist;       // [Q][4096], filled by the indexer or by launch_topk_hist
  uint32_t* counters;   // [Q][8]: [0],[1] append cursors (zero on entry), [4..6] threshold record
  int32_t* sel;         // [Q][k]
  uint2* cand;          // [Q][cand_cap]
  int64_t cand_cap;
  // single-block path only: 0 = n_vis array; 1 = decode (n_vis = ctx_len/4, also writes the ring
  // window into idx[-128..-1]); 2 = causal prefill from pos0 (also writes the raw window)
  int win_mode;
  const int32_t* ctx_len;
  int64_t max_ctx;
  int64_t pos0;
  int q_per_req = 1;    // decode: queries per request (the last q_per_req tokens of each request)
  int ring = 128;       // decode: window ring slots per request (slot = position % ring)
  // single-block path only, optional: also write each selected entry's compressed KV row
  // (page_table[request][idx >> 6] * 64 + (idx & 63), -1 if unmapped) to rows[q * ld_rows + j]
  int32_t* rows;
  int64_t ld_rows;
  const int32_t* page_table;
  int max_pages;
  int num_pages;
  // sketch path only: the indexer's per-wave sketches of each row (see IndexerArgs)
  const uint2* sk_top = nullptr;
  const uint32_t* sk_bound = nullptr;
  int64_t sk_waves = 0;
  // sketch path only: the indexer launch of this decode; rows with at least ia.sk_rescore_from
  // visible entries (> 0) have no stored scores and are rescored when their sketches cannot decide
  IndexerArgs ia{};
};
hipError_t launch_topk_hist(const TopkArgs& a, hipStream_t s);
hipError_t launch_topk_select(const TopkArgs& a, hipStream_t s);
hipError_t launch_topk_single(const TopkArgs& a, hipStream_t s);
bool topk_single_ok(int64_t max_n_vis, int k);
// Long rows of a decode (one or several queries per request): the indexer writes per-wave sketches (8 largest
// scores of every 512 entries and a bound on the rest) and one block per query selects from them.
hipError_t launch_topk_sketch(const TopkArgs& a, hipStream_t s);
bool topk_sketch_ok(int64_t max_n_vis, int k);
int64_t topk_sketch_waves(int64_t max_n_vis);   // sketches per row
// visible entries from which a sketch row is sure to hold k real sketch entries
int64_t sketch_rescore_from(int k);

// Zero histograms / counters and write window indices (decode ring or causal prefill window).
struct PrepArgs {
  uint32_t* zero_ptr;        // words to clear
  int64_t zero_words;
  int mode;                  // 0: none, 1: decode ring, 2: causal prefill
  int rows;                  // B (decode) or Q (prefill)
  const int32_t* ctx_len;    // decode: [B]
  int64_t max_ctx;           // decode: clamp of ctx_len
  int64_t pos0;              // prefill: position of query 0
  int32_t* idx;              // [rows][ld_idx] window part written to columns [0,128)
  int64_t ld_idx;
  int32_t* n_vis_out;        // [rows]
  int32_t* q_req_out;        // optional [rows]: request id of each row (decode: row, prefill: 0)
  int ratio;                 // raw tokens per compressed entry: n_vis = T / ratio or (t + 1) / ratio
  int q_per_req = 1;         // decode: queries per request (row = request * q_per_req + token)
  int ring = 128;            // decode: window ring slots per request (slot = position % ring)
  int64_t comp_cols;         // > 0: also write compressed columns [128, 128 + comp_cols) as j < n_vis ? j : -1
};
hipError_t launch_prep(const PrepArgs& a, hipStream_t s);

struct AttnArgs {
  const void* q;             // [Q][H][512]
  int q_dt;                  // 0 f32, 1 bf16
  int Q, H;
  const float* sink;
  const uint8_t* win;
  int win_fmt;
  int64_t win_rows_per_req;
  const uint8_t* comp;
  int comp_fmt;
  int comp_num_pages;
  const int32_t* page_table;
  int max_pages;
  const int32_t* q_req;
  int n_req;
  const int32_t* idx;
  int64_t ld_idx;
  int n_win, n_comp;
  float softmax_scale;
  void* out;
  int out_dt;                // 0 f32, 1 bf16
  float* part;               // split-K partials (may be null when n_split == 1)
  int n_split;               // chosen by plan_attn_split
  int tiles_per_split = 0;   // 32-slot tiles per split (set by launch_attention)
  int req_mode;              // 0: q_req array; 1: request = query / q_per_req (decode); 2: request 0 (prefill)
  int q_per_req = 1;
  // causal prefill (req_mode 2) from a fused path: compressed slots at or past
  // min(n_comp, (pos0 + q + 1) / trim_ratio) are known to be invalid (0: no such knowledge)
  int trim_ratio = 0;
  int64_t pos0 = 0;
  // no row is gathered for two queries (decode, one query per request): rows are streamed with
  // non-temporal loads
  bool stream_rows = false;
  // optional: compressed slot j of query q is row rows[q * ld_rows + j] of the pool (< 0 invalid),
  // already resolved through the page table; null = resolve idx through the page table
  const int32_t* rows;
  int64_t ld_rows;
  // host side only, optional (one-query-per-request decode with one-block rows): the selection of
  // this step.  launch_attention either runs it inside the 64-head attention blocks (each block
  // selects its query's rows into LDS, and the blocks of split 0 also write idx / rows) or launches
  // it first.
  const struct TopkArgs* sel = nullptr;
};
struct CompressArgs {
  const void* kv;            // token projections, row (tok - tok0) at kv + row * ld: [n_tok][coff * D]
  const void* score;         // gate projections, same layout
  int proj_dt;               // 0 f32, 1 bf16
  int64_t ld;                // elements per projection row
  int64_t tok0;              // raw position of projection row 0
  int ratio;                 // 4 (overlapping windows, coff = 2) or 128 (coff = 1)
  int D;                     // 512 (KV rows) or 128 (indexer keys)
  const float* ape;          // [ratio][coff * D]
  const float* norm_w;       // [D]
  float eps;
  const float* rope_cos;     // [c_count][32]
  const float* rope_sin;
  int64_t c_begin;
  int c_count;
  uint8_t* out;              // KV pool rows (D = 512) or indexer key bytes (D = 128)
  int out_fmt;               // D = 512: row format 0/1/2; D = 128: 2 fp8, 3 fp4
  uint8_t* out_scales;       // D = 128: [P][4][64] E8M0
  int num_pages;
  const int32_t* page_table; // the request's row
};
hipError_t launch_compress(const CompressArgs& a, hipStream_t s);

int plan_attn_split(int Q, int H, int n_idx, int q_dt);
int attn_head_block(int Q, int H, int n_idx);   // 16 or 64 heads per block of the matrix-core kernels
// true when the BF16 matrix-core kernel serves this call (bf16 q, BF16/FP8 rows); else the fp32 kernel
bool attn_uses_matrix_cores(int q_dt, int win_fmt, int comp_fmt, int n_win, int n_comp);
size_t attn_partial_bytes(int Q, int H, int n_idx);
hipError_t launch_attention(const AttnArgs& a, hipStream_t s);

}  // namespace csa
