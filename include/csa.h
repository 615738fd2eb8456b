/*
 * csa.h - C ABI of the compressed-sparse-attention (CSA) hot path on AMD Instinct MI355X (gfx950).
 *
 * The path computes, for each query token:
 *   (1) indexer scores of every visible 4:1-compressed entry,
 *         s[c] = sum_h w[h] * max(0, qI[h] . kI[c])
 *       with FP8 E4M3FN indexer queries/keys carrying one E8M0 scale per 32 elements;
 *   (2) the indices of the top-k scores (k = 512 in the model);
 *   (3) sparse multi-query attention over [sliding-window rows ++ selected compressed rows]:
 *         out[h] = sum_j e^{S[h,j]} v_j / (sum_j e^{S[h,j]} + e^{sink[h]}),  S = scale * q[h] . v_j
 *       where K and V are the same single-head 512-dim rows and invalid index slots are skipped.
 * Around that path the library also provides: MXFP4 (E2M1) indexer operands (CSA_FP4_E2M1),
 * decode steps that take several tokens of each request at once (csa_decode_multi), layers whose
 * compressed cache has no indexer and is attended whole (csa_hca_decode / csa_hca_prefill), and
 * the compressor that writes both caches (csa_compress_kv / csa_compress_index_keys).
 *
 * Sources (pages as titled; the section is named on each declaration):
 *   [P1] "DeepSeek-V4 全面解读：架构设计与 inference/encoding 源码深度解析" (wangjunjian.com)
 *   [P2] "DeepSeek-V4 in SGLang 深度理解分析" (kenforever1.github.io)
 *   [P3] "tilelang量化内核拆解DeepSeek-V4.1-Flash-NVFP4的fp4_gemm与sparse_attn实现" (wzjinhao.cn)
 *
 * Conventions shared by every entry point
 *   - All data pointers are DEVICE pointers owned by the caller.  The library never allocates,
 *     frees or retains them; work is enqueued on `stream` and nothing is synchronised.  Keep the
 *     buffers alive until the stream work has completed.
 *   - Scratch memory ("ws") is caller-provided and sized by the matching *_workspace_bytes query.
 *     Its contents on entry do not matter; the entry point initialises what it uses.
 *   - Arguments are validated on the host before anything is launched; on error nothing is written
 *     and nothing is enqueued.  Device-resident *values* (indices, page ids, lengths, request ids)
 *     are data: out-of-range values are masked exactly like the -1 slot, never dereferenced.
 *   - Every device pointer must be 16-byte aligned (CSA_ERR_ALIGN otherwise).
 *   - Layouts are C order.  D = 512 (448 "nope" dims then 64 "rope" dims, rope last as in [P1]
 *     section 2.11 step 8), DI = 128 indexer dims, a page holds 64 consecutive compressed entries.
 *   - Calls on different streams may run concurrently; calls that share a workspace must not.
 */
#ifndef CSA_H
#define CSA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CSA_OK = 0,
  CSA_ERR_NULL = -1,        /* a required pointer is NULL                                      */
  CSA_ERR_SHAPE = -2,       /* a size is out of its documented range                            */
  CSA_ERR_DTYPE = -3,       /* unknown or unsupported dtype / format code                       */
  CSA_ERR_ALIGN = -4,       /* a pointer is not 16-byte aligned                                 */
  CSA_ERR_WORKSPACE = -5,   /* ws is NULL or smaller than the *_workspace_bytes query            */
  CSA_ERR_UNSUPPORTED = -6, /* a valid combination the library does not implement             */
  CSA_ERR_HIP = -7,         /* a HIP launch failed; csa_last_hip_error() holds the hipError_t   */
  CSA_ERR_SCRATCH = -8      /* csa_decode_noalloc: the call needs more than its static scratch  */
} csa_status;

/* Element types of q, out and the indexer operands. */
/* CSA_FP4_E2M1 packs two E2M1 codes per byte: element 2i in bits [0,4), element 2i+1 in bits
 * [4,8) (code = sign bit 3 | exponent bits 2..1 | mantissa bit 0, magnitudes 0, 0.5, 1, 1.5, 2, 3,
 * 4, 6), as the block FP4 quantiser of [P1] section 3.5 writes them.  Indexer operands only.    */
typedef enum { CSA_F32 = 0, CSA_BF16 = 1, CSA_FP8_E4M3FN = 2, CSA_FP4_E2M1 = 3 } csa_dtype;

/* KV row formats (one 512-dim row each).
 *   CSA_KV_F32               2048 B: 512 x fp32
 *   CSA_KV_BF16              1024 B: 512 x bf16
 *   CSA_KV_FP8NOPE_BF16ROPE   608 B: [0,448) e4m3fn nope | [448,576) 64 x bf16 rope |
 *                                   [576,604) 7 x fp32 scale, one per 64 nope dims | [604,608) pad
 *     value of nope dim i = fp8(byte i) * scale[i / 64]            ([P2] concept 5)          */
typedef enum { CSA_KV_F32 = 0, CSA_KV_BF16 = 1, CSA_KV_FP8NOPE_BF16ROPE = 2 } csa_kv_format;

/* Paged compressed KV pool.  Entry c of request r lives in row
 *   page_table[r * max_pages + (c >> 6)] * 64 + (c & 63)   of `rows` ([num_pages][64][row bytes]).
 * A page id outside [0, num_pages) masks the entry.                                          */
typedef struct {
  const void* rows;
  int32_t fmt;              /* csa_kv_format */
  int32_t num_pages;
  const int32_t* page_table;/* [n_req][max_pages] */
  int32_t max_pages;
  int32_t reserved;
} csa_paged_kv;

/* Paged indexer key cache (same page mapping as csa_paged_kv).
 *   dt = CSA_FP8_E4M3FN: keys [num_pages][8192] e4m3fn bytes, one page of 64 slots x 128 dims in
 *        operand order (below); scales [num_pages][4][64] E8M0 bytes, scales[p][b][s] scaling
 *        dims [32b, 32b+32) of slot s (value 2^(e-127)).
 *   dt = CSA_FP4_E2M1: keys [num_pages][4096] bytes (64 slots x 64 bytes, two E2M1 codes per
 *        byte) in operand order; scales as for CSA_FP8_E4M3FN (one E8M0 byte per 32 dims).
 *   dt = CSA_F32: keys [num_pages][64][128] fp32, row-major; scales must be NULL.
 * Operand order: with R = 128 (FP8) or 64 (FP4) bytes per slot and halves = R / 64, byte b of
 * slot s sits at page byte ((s % 4) * halves + b / 64) * 1024 + (s / 4 + 16 * ((b % 64) / 16)) * 16
 * + b % 16.  Each kilobyte of a page is then one 16-byte chunk for each of the 64 lanes of a
 * matrix-core operand, so the indexer reads every page with contiguous 1 KB loads.
 * csa_compress_index_keys writes this order; pack_index_keys() in the Python package converts
 * row-major [P][64][R] bytes to it.                                                            */
typedef struct {
  const void* keys;
  const uint8_t* scales;
  int32_t dt;               /* csa_dtype: CSA_FP8_E4M3FN, CSA_FP4_E2M1 or CSA_F32 */
  int32_t num_pages;
  const int32_t* page_table;/* [n_req][max_pages] */
  int32_t max_pages;
  int32_t reserved;
} csa_paged_idx;

/* ---------------------------------------------------------------------------------------------
 * csa_indexer_logits - indexer scores ([P1] section 2.10 forward steps 5-8; [P2] concept 3 and
 * algorithm 2, the FP8 "paged MQA logits" pass).
 *
 *   qI        [Q][HI][128] e4m3fn bytes (qI_dt = CSA_FP8_E4M3FN), [Q][HI][64] bytes of packed
 *             E2M1 pairs (CSA_FP4_E2M1) or [Q][HI][128] fp32 (CSA_F32)
 *   qI_scale  [Q][HI][4] E8M0 bytes, one per 32 dims (NULL for CSA_F32)
 *   w         [Q][HI] fp32 head weights (the caller folds softmax_scale * HI^-0.5 into them)
 *   keys      paged indexer keys; the key dtype must equal qI_dt
 *   q_req     [Q] request id of each query (row of the page table), n_req requests
 *   n_vis     [Q] visible compressed entries of each query (decode: T/4; causal prefill at raw
 *             position t: (t+1)/4).  Clamped to [0, min(max_n_vis, 64*max_pages)].
 *   logits    [Q][ld] fp32 out: s[c] for c < n_vis[q], -INFINITY for n_vis[q] <= c < max_n_vis;
 *             columns >= max_n_vis are not written.
 * Arithmetic: every product of two dequantised codes is exact and the dot products accumulate in
 * fp32 (FP8 codes are converted exactly to bf16 with their block scales folded in; E2M1 products
 * are exact on the FP4 matrix cores), then ReLU, the weights and the head sum in fp32.  FP8 scale
 * bytes must lie in [10, 245] (an FP8 value times its scale is then a normal bf16); 0xFF (NaN)
 * is not supported.
 * Ranges: 1 <= Q, 1 <= HI <= 64, 0 <= max_n_vis <= ld, n_req >= 1.
 * ------------------------------------------------------------------------------------------- */
csa_status csa_indexer_logits(const void* qI, const uint8_t* qI_scale, int32_t qI_dt,
                              const float* w, const csa_paged_idx* keys,
                              const int32_t* q_req, int32_t n_req, const int32_t* n_vis,
                              int32_t Q, int32_t HI, int64_t max_n_vis,
                              float* logits, int64_t ld, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * csa_topk - per-query top-k selection over the visible prefix of each logits row ([P1] section
 * 2.10 steps 9-10 with the visibility mask applied first; [P2] concept 3, top-512).
 *
 *   logits    [Q][ld] fp32; only columns c < n_vis[q] (clamped to [0, max_n_vis]) are candidates
 *   idx       [Q][ld_idx] int32 out, first k columns written:
 *               n_vis <= k : 0, 1, ..., n_vis-1, then -1 padding;
 *               n_vis  > k : the k candidates with the largest scores, equal scores ordered by
 *                            ascending index, written in ascending index order.
 *             NaN scores rank below -INFINITY; -0.0 equals +0.0.
 *   ws        >= csa_topk_workspace_bytes(Q, max_n_vis, k) bytes
 * Ranges: 1 <= Q, 1 <= k <= 2048, 0 <= max_n_vis <= ld, ld_idx >= k.
 * ------------------------------------------------------------------------------------------- */
size_t csa_topk_workspace_bytes(int32_t Q, int64_t max_n_vis, int32_t k);
csa_status csa_topk(const float* logits, int64_t ld, const int32_t* n_vis, int32_t Q,
                    int64_t max_n_vis, int32_t k, int32_t* idx, int64_t ld_idx,
                    void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * csa_sparse_attn - index-gathered multi-query attention with a per-head sink ([P1] section 3.7,
 * sparse_attn_kernel: gather by index, online softmax, sink added to the denominator after the
 * loop; [P3] sparse_attn section: running max starts at -1e30 so an all-invalid row gives 0).
 *
 *   q         [Q][H][512], q_dt CSA_BF16 (BF16 matrix-core path, fp32 accumulation) or CSA_F32
 *             (fp32 path)
 *   sink      [H] fp32 (not multiplied by softmax_scale)
 *   win_rows  [n_req][win_rows_per_req][row bytes of win_fmt]: the window source (a 128-slot ring
 *             at decode, the raw rows of the request at prefill); may be NULL when n_win == 0
 *   comp      the paged compressed KV (may be NULL when n_comp == 0)
 *   q_req     [Q] request id of each query
 *   idx       [Q][ld_idx] int32: columns [0, n_win) index the window source of the query's request,
 *             columns [n_win, n_win+n_comp) index compressed entries.  Negative or out-of-range
 *             values (and unmapped pages) are invalid slots.  Duplicates count once per slot.
 *   out       [Q][H][512], out_dt CSA_BF16 or CSA_F32; a query with no valid slot gets exact 0.
 *   ws        >= csa_sparse_attn_workspace_bytes(Q, H, n_win + n_comp) bytes (split-K partials)
 * Ranges: 1 <= Q, 1 <= H <= 128, 0 <= n_win, 0 <= n_comp, 1 <= n_win + n_comp <= 16384,
 *         ld_idx >= n_win + n_comp, softmax_scale finite.
 * ------------------------------------------------------------------------------------------- */
size_t csa_sparse_attn_workspace_bytes(int32_t Q, int32_t H, int32_t n_idx);
csa_status csa_sparse_attn(const void* q, int32_t q_dt, int32_t Q, int32_t H, const float* sink,
                           const void* win_rows, int32_t win_fmt, int64_t win_rows_per_req,
                           const csa_paged_kv* comp, const int32_t* q_req, int32_t n_req,
                           const int32_t* idx, int64_t ld_idx, int32_t n_win, int32_t n_comp,
                           float softmax_scale, void* out, int32_t out_dt,
                           void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * csa_decode - one decode step of B requests (one query each) through the whole path: indexer
 * scores -> top-k -> [window ++ top-k] -> sparse attention ([P1] section 2.11 forward steps 3-7).
 *
 *   ctx_len   [B] raw context length T_b including the current token (device).  The query sees
 *             n_vis = T_b / 4 compressed entries and the last min(T_b, 128) raw tokens, which live
 *             in ring slots (position % 128) of win_ring ([P1] section 2.8, decode ring buffer).
 *   max_ctx   host-side upper bound of ctx_len (sizes the workspace); larger values are clamped.
 *   win_ring  [B][128][row bytes of win_fmt]
 *   idx_out   optional [B][128 + k] int32: the index list attended ([window slots ++ top-k]);
 *             NULL to keep it in the workspace only.
 *   Other arguments as in the primitives above (q_req is the identity).
 * Ranges: 1 <= B, 1 <= H <= 128, 1 <= HI <= 64, 1 <= k <= 2048, 0 <= max_ctx <= 2^31-1.
 * ------------------------------------------------------------------------------------------- */
size_t csa_decode_workspace_bytes(int32_t B, int32_t H, int32_t HI, int64_t max_ctx, int32_t k);
csa_status csa_decode(int32_t B, int32_t H, int32_t HI, int32_t k,
                      const void* q, int32_t q_dt, const float* sink,
                      const void* qI, const uint8_t* qI_scale, int32_t qI_dt, const float* w,
                      const csa_paged_idx* keys, const csa_paged_kv* comp,
                      const void* win_ring, int32_t win_fmt,
                      const int32_t* ctx_len, int64_t max_ctx,
                      float softmax_scale, void* out, int32_t out_dt, int32_t* idx_out,
                      void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * csa_decode_noalloc - csa_decode for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the same arguments and
 * result, minus the workspace, which comes from a static device array of CSA_NOALLOC_SCRATCH_BYTES
 * compiled into the library (each device the library runs on holds its own copy until the
 * process ends).  The call allocates nothing and calls no allocating routine.
 *   Limit: calls whose csa_decode_workspace_bytes(B, H, HI, max_ctx, k) exceeds
 *   CSA_NOALLOC_SCRATCH_BYTES return CSA_ERR_SCRATCH before anything is enqueued.
 *   The stream must belong to the current device.  Every call on a device shares that device's
 *   array, which keeps the last call's contents: calls that overlap on one device (different
 *   streams or host threads without ordering between them) race and must not be issued.
 * Errors as csa_decode, plus CSA_ERR_SCRATCH, and CSA_ERR_HIP if the array's address cannot be
 * obtained on the current device.
 * ------------------------------------------------------------------------------------------- */
#define CSA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
csa_status csa_decode_noalloc(int32_t B, int32_t H, int32_t HI, int32_t k,
                              const void* q, int32_t q_dt, const float* sink,
                              const void* qI, const uint8_t* qI_scale, int32_t qI_dt, const float* w,
                              const csa_paged_idx* keys, const csa_paged_kv* comp,
                              const void* win_ring, int32_t win_fmt,
                              const int32_t* ctx_len, int64_t max_ctx,
                              float softmax_scale, void* out, int32_t out_dt, int32_t* idx_out,
                              hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * csa_decode_multi - a decode step that takes the last S tokens of each of B requests at once
 * (multi-token prediction / speculative decoding: [P1] section 2.17 MTPBlock, [P2]'s NextN
 * variant), through the same path as csa_decode.  Query b*S + j sits at position T_b - S + j and
 * sees what a one-query decode with context T_b - (S - 1 - j) would: n_vis = (T_b - S + j + 1) / 4
 * compressed entries and the 128 raw tokens up to its position.
 *
 *   q, qI, qI_scale, w, out   B*S query rows, request-major (row b*S + j)
 *   win_ring   [B][ring_slots][row bytes of win_fmt]: raw token p of request b in slot p % ring_slots;
 *              ring_slots >= 128 + S - 1 keeps the earliest query's window in the ring
 *   idx_out    optional [B*S][128 + k] int32
 *   Other arguments as in csa_decode; S = 1 with ring_slots = 128 is exactly csa_decode.
 * Ranges: 1 <= S <= 16, B*S <= 65535, 128 + S - 1 <= ring_slots <= 2^20, others as csa_decode.
 * ------------------------------------------------------------------------------------------- */
size_t csa_decode_multi_workspace_bytes(int32_t B, int32_t S, int32_t H, int32_t HI, int64_t max_ctx, int32_t k);
csa_status csa_decode_multi(int32_t B, int32_t S, int32_t H, int32_t HI, int32_t k,
                            const void* q, int32_t q_dt, const float* sink,
                            const void* qI, const uint8_t* qI_scale, int32_t qI_dt, const float* w,
                            const csa_paged_idx* keys, const csa_paged_kv* comp,
                            const void* win_ring, int32_t win_fmt, int32_t ring_slots,
                            const int32_t* ctx_len, int64_t max_ctx,
                            float softmax_scale, void* out, int32_t out_dt, int32_t* idx_out,
                            void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * csa_prefill - causal prefill of one request: Q queries at raw positions pos0 .. pos0+Q-1.
 * Query t sees compressed entries c < (t+1)/4 and raw rows [t-127, t] of raw_rows ([P1] section
 * 2.8, causal window at prefill; section 2.10 causal mask).  Page tables have one row.
 *
 *   raw_rows  [T][row bytes of raw_fmt], the request's raw KV rows (window source)
 *   idx_out   optional [Q][128 + k] int32 as in csa_decode
 * Ranges: 1 <= Q, 0 <= pos0, pos0 + Q <= T, 1 <= H <= 128, 1 <= HI <= 64, 1 <= k <= 2048.
 * ------------------------------------------------------------------------------------------- */
size_t csa_prefill_workspace_bytes(int32_t Q, int32_t H, int32_t HI, int64_t T, int32_t k);
csa_status csa_prefill(int32_t Q, int32_t H, int32_t HI, int32_t k,
                       const void* q, int32_t q_dt, const float* sink,
                       const void* qI, const uint8_t* qI_scale, int32_t qI_dt, const float* w,
                       const csa_paged_idx* keys, const csa_paged_kv* comp,
                       const void* raw_rows, int32_t raw_fmt, int64_t T, int64_t pos0,
                       float softmax_scale, void* out, int32_t out_dt, int32_t* idx_out,
                       void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * csa_hca_decode / csa_hca_prefill - attention layers whose compressed cache has no indexer (the
 * heavily compressed C128 layers of [P1]'s hybrid CSA/HCA design; [P1] section 2.8
 * get_compress_topk_idxs and the attention forward's branch without an indexer, [P2] concept 2).
 * Each query attends [window ++ every visible compressed entry]: with `ratio` raw tokens per
 * compressed entry, decode sees n_vis = T_b / ratio entries and prefill query t sees (t+1) / ratio.
 * The window is as in csa_decode (ring of the last 128 tokens) and csa_prefill (raw rows
 * [t-127, t]).  The attention, its precision and its output are those of csa_sparse_attn.
 *
 *   comp      paged compressed KV; entry c of request r lives at page_table[r][c >> 6], slot c & 63
 *   ratio     raw tokens per compressed entry (128 for C128; any value >= 1)
 *   ws        >= csa_hca_decode_workspace_bytes(B, H, max_ctx, ratio) (decode) or
 *             csa_hca_prefill_workspace_bytes(Q, H, T, ratio) (prefill) bytes: the index lists
 *             and split-K partials.  The workspace functions return 0 for arguments out of range.
 *   Other arguments as in csa_decode / csa_prefill (no indexer inputs, no top-k).
 * Ranges: as csa_decode / csa_prefill, plus 1 <= ratio and 128 + min(max_ctx / ratio,
 *         64 * comp->max_pages) <= 16384 (decode; prefill with (pos0 + Q) / ratio).
 * ------------------------------------------------------------------------------------------- */
size_t csa_hca_decode_workspace_bytes(int32_t B, int32_t H, int64_t max_ctx, int32_t ratio);
csa_status csa_hca_decode(int32_t B, int32_t H, const void* q, int32_t q_dt, const float* sink,
                          const csa_paged_kv* comp, const void* win_ring, int32_t win_fmt,
                          const int32_t* ctx_len, int64_t max_ctx, int32_t ratio,
                          float softmax_scale, void* out, int32_t out_dt,
                          void* ws, size_t ws_bytes, hipStream_t stream);
size_t csa_hca_prefill_workspace_bytes(int32_t Q, int32_t H, int64_t T, int32_t ratio);
csa_status csa_hca_prefill(int32_t Q, int32_t H, const void* q, int32_t q_dt, const float* sink,
                           const csa_paged_kv* comp, const void* raw_rows, int32_t raw_fmt,
                           int64_t T, int64_t pos0, int32_t ratio,
                           float softmax_scale, void* out, int32_t out_dt,
                           void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * csa_compress_kv / csa_compress_index_keys - the compressor that fills the caches this path
 * reads ([P1] section 2.9 Compressor, 2.6 apply_rotary_emb, 2.7 rotate_activation; [P2] concept
 * 2).  Entries c_begin .. c_begin+c_count-1 of one request are computed and written to page
 * page_table_row[c >> 6], slot c & 63 (unmapped pages are skipped).
 *
 *   kv_proj, score_proj  the token projections of the kv and gate linear maps (computed by the
 *             caller): row (p - tok0) at ptr + row * ld_proj holds raw token p, coff * D
 *             elements, proj_dt CSA_BF16 or CSA_F32.  coff = 2 at ratio 4 (each token's
 *             overlapping half [0, D) serves the next window, its normal half [D, 2D) its own
 *             window), 1 at ratio 128.  Entry c pools tokens [c*ratio, (c+1)*ratio) and, at ratio 4
 *             with c > 0, the overlapping halves of tokens [(c-1)*4, c*4); those rows must lie in
 *             [tok0, tok0 + n_tok).
 *   ape       [ratio][coff * D] fp32 position embedding added to the gate scores
 *   norm_w    [D] fp32 RMSNorm weight; eps its epsilon
 *   rope_cos, rope_sin  [c_count][32] fp32: the rotary angles of each entry (row i: entry
 *             c_begin + i); pairs (2j, 2j+1) of the last 64 features are rotated by angle j
 *   Per entry and feature: softmax over the window positions of (score + ape), weighted sum of
 *   kv; RMSNorm over the D features; rotary embedding.
 * csa_compress_kv: D = 512; pool_rows [num_pages][64][row bytes] in pool_fmt (csa_kv_format):
 *   FP8NOPE_BF16ROPE rows quantise the 448 nope features per 64 with scale max(amax,1e-4)/448.
 * csa_compress_index_keys: D = 128, then the scaled Hadamard rotation of the row, then key_dt
 *   CSA_FP8_E4M3FN (keys: 8 KB pages) or CSA_FP4_E2M1 (4 KB pages), in the operand order of
 *   csa_paged_idx, with one E8M0 scale
 *   per 32 features in scales [P][4][64]: 2^ceil(log2(max(amax,1e-4)/448)) for FP8,
 *   2^ceil(log2(max(amax,6*2^-126)/6)) for FP4.
 * Ranges: ratio 4 or 128; ld_proj >= coff * D, a multiple of 8; c_begin + c_count <= 64 *
 *         max_pages; eps >= 0.  Projections, ape, norm_w, rope tables and outputs 16-byte aligned.
 * ------------------------------------------------------------------------------------------- */
csa_status csa_compress_kv(const void* kv_proj, const void* score_proj, int32_t proj_dt, int64_t ld_proj,
                           int64_t tok0, int64_t n_tok, int32_t ratio, const float* ape, const float* norm_w,
                           float eps, const float* rope_cos, const float* rope_sin,
                           int64_t c_begin, int32_t c_count, void* pool_rows, int32_t pool_fmt,
                           int32_t num_pages, const int32_t* page_table_row, int32_t max_pages,
                           hipStream_t stream);
csa_status csa_compress_index_keys(const void* kv_proj, const void* score_proj, int32_t proj_dt,
                                   int64_t ld_proj, int64_t tok0, int64_t n_tok, int32_t ratio,
                                   const float* ape, const float* norm_w, float eps,
                                   const float* rope_cos, const float* rope_sin,
                                   int64_t c_begin, int32_t c_count, void* keys, uint8_t* scales,
                                   int32_t key_dt, int32_t num_pages, const int32_t* page_table_row,
                                   int32_t max_pages, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * Diagnostics.
 *   csa_status_string   static text of a status code.
 *   csa_last_hip_error  hipError_t of the last CSA_ERR_HIP on the calling thread (0 if none).
 *   csa_profile_enable  on != 0: every kernel the entry points launch carries a pair of hipEvents
 *                       attached to its own dispatch (hipExtLaunchKernelGGL), which time the
 *                       kernel's execution on the GPU; adds no synchronisation.
 *   csa_profile_collect synchronises the recorded events and returns, for the kernel named
 *                       `kernel` (e.g. "indexer_fp8"), the summed duration in ms and the number
 *                       of launches since the last reset; unknown names return 0 launches.
 *   csa_profile_reset   forgets all recorded events.
 *   csa_debug_violations  debug builds (compiled with -DCSA_DEBUG_CHECKS): the number of device-
 *                       resident values the kernels masked as invalid since the last call (an
 *                       index that is not -1 but lies at or past its source or on an unmapped page,
 *                       a visible indexer page with no page id in the pool), then clears it; read
 *                       after the work is complete (synchronise first).  Release builds return
 *                       CSA_ERR_UNSUPPORTED with *count = 0.
 * Profiling state is process-wide (a diagnostic, the library's only mutable state apart from the
 * scratch array of csa_decode_noalloc and the debug counters), guarded by a mutex.
 * ------------------------------------------------------------------------------------------- */
const char* csa_status_string(int32_t status);
int32_t csa_last_hip_error(void);
csa_status csa_debug_violations(uint64_t* count);
csa_status csa_profile_enable(int32_t on);
csa_status csa_profile_collect(const char* kernel, double* total_ms, int64_t* launches);
csa_status csa_profile_reset(void);

#ifdef __cplusplus
}
#endif
#endif /* CSA_H */
