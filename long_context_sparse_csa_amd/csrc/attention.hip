// Index-gathered multi-query attention with a per-head sink on gfx950.
//
// What is computed follows [P1] "DeepSeek-V4 全面解读" section 3.7 (sparse_attn_kernel): rows are
// gathered by index, -1 slots are masked, scores are scale * q.kv, an online softmax keeps a running
// max and sum, P.V accumulates, and after the loop e^(sink - max) joins the denominator.  [P3]
// "tilelang量化内核拆解…" (sparse_attn section) fixes the running-max start at the finite -1e30, so a
// query with no valid slot outputs exact zeros.  K and V are the same 512-dim rows.
//
// BF16 matrix-core kernel (q bf16): a block owns one query, up to 64 heads (four head groups of
// 16) and a contiguous range of 32-slot tiles (at most 1024 slots; longer lists are split).  Eight
// waves in two roles share each SIMD.  Score wave w holds q of head groups w and w ^ 1 over one
// half of the dims, so each K fragment it reads feeds two MFMAs and every K element is read by two
// waves; the partial scores of group w ^ 1 go to wave w ^ 1 through LDS, and wave w runs the online
// softmax of group w.  Value wave 4 + w accumulates output dims [128w, 128w+128) of all 64 heads.
// Every wave resolves and gathers four rows of each tile (coalesced: one 16-B lane chunk per 8 dims
// of a row, FP8 nope dequantised with its fp32 block scale) into a ring of four row-major bf16 LDS
// tiles.  Scores are computed transposed (S^T = K.q^T) so each lane holds 8 scores of its own head;
// once the key order inside the 32-wide K step is permuted (slot 8g+4mt+i <-> key 16mt+4g+i) these
// are exactly the P^T operand of O^T = V^T.P^T, which the value waves read from LDS.  They read V^T
// from the same row-major tile with gfx950's transposing LDS load (ds_read_b64_tr_b16): each V
// fragment feeds four MFMAs and no transposed copy is ever written.  The roles run a tile apart
// (the scores of tile p, the softmax of tile p - 1 and P.V of tile p - 2 share one phase), one
// barrier per tile.  Softmax runs in base 2 with log2(e) folded into the scale.  Large
// queries-by-heads grids run unsplit; small ones split the slot range across blocks and a combine
// kernel merges the (max, sum, acc) partials, sink included.
//
// fp32 kernel (q f32): one block per (query, head); scores, softmax and P.V in fp32 with natural
// exp, for bit-accurate-ish comparisons against the fp64 definition.
#include <cstdlib>

#include "attn_common.h"
#include "indexer_score.h"
#include "select_block.h"

namespace csa {


struct RowSrc {
  const uint8_t* p;
  int fmt;
};

// Resolve slot s of query q's index list to a row address (nullptr = invalid slot).
__device__ __forceinline__ RowSrc resolve_slot(const AttnArgs& a, int q, int r, int s) {
  RowSrc rs{nullptr, 0};
  if (r < 0 || r >= a.n_req || s >= a.n_win + a.n_comp) return rs;
  const int v = a.idx[(int64_t)q * a.ld_idx + s];
  if (v < 0) return rs;
  if (s < a.n_win) {
    if (a.win != nullptr && v < a.win_rows_per_req) {
      rs.p = a.win + ((int64_t)r * a.win_rows_per_req + v) * row_bytes(a.win_fmt);
      rs.fmt = a.win_fmt;
    }
  } else if (a.comp != nullptr && (int64_t)v < (int64_t)a.max_pages * kPage) {
    const int pg = a.page_table[(int64_t)r * a.max_pages + (v >> 6)];
    if ((unsigned)pg < (unsigned)a.comp_num_pages) {
      rs.p = a.comp + ((int64_t)pg * kPage + (v & 63)) * row_bytes(a.comp_fmt);
      rs.fmt = a.comp_fmt;
    }
  }
  CSA_DBG_COUNT(rs.p == nullptr);   // an index that is not -1 yet has no row
  return rs;
}

// Dims [8*dc, 8*dc+8) of a row, dequantised to fp32.
__device__ __forceinline__ void load_chunk8(const uint8_t* row, int fmt, int dc, float* v) {
  if (row == nullptr) {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = 0.f;
    return;
  }
  if (fmt == kRowBF16) {
    const uint4 x = *(const uint4*)(row + 16 * dc);
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = __uint_as_float(w[e] << 16);
      v[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
    }
  } else if (fmt == kRowF32) {
    const float4 x = *(const float4*)(row + 32 * dc);
    const float4 y = *(const float4*)(row + 32 * dc + 16);
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
    v[4] = y.x; v[5] = y.y; v[6] = y.z; v[7] = y.w;
  } else if (dc < kNope / 8) {
    const uint2 x = *(const uint2*)(row + 8 * dc);
    const float sc = *(const float*)(row + 576 + 4 * (dc >> 3));
    fp8x4_to_f32(x.x, v);
    fp8x4_to_f32(x.y, v + 4);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] *= sc;
  } else {
    const uint4 x = *(const uint4*)(row + 448 + 16 * (dc - kNope / 8));
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = __uint_as_float(w[e] << 16);
      v[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
    }
  }
}

// Two 8-byte loads per lane per row, without branches, so a whole tile of loads is in flight at
// once.  Lane dc covers dims [8dc, 8dc+8).  BF16 rows: the two halves of the lane's 16 bytes.  FP8
// rows: nope lanes (dc < 56) take their 8 e4m3fn codes and, in the second load, the 8-byte aligned
// pair of fp32 block scales that holds the scale of their 64-dim block; rope lanes (dc >= 56) take
// the two halves of 8 bf16 values.  The code is wave-uniform, so the row address is scalar.
struct RawChunk {
  v2u lo, hi;
};

// NTG: non-temporal loads, for paths where no row is read by two queries (decode with one query per
// request); a prefill re-reads each row for many queries and keeps the cached loads
template <int WF, int CF, bool NTG>
__device__ __forceinline__ RawChunk load_raw(uint64_t code, int dc) {
  const int fmt = (code & kCodeComp) ? CF : WF;
  const gbytes rp = (gbytes)(uintptr_t)(code & kCodeAddrMask);
  int o0 = 16 * dc, o1 = 16 * dc + 8;
  if (fmt == kRowFP8) {
    const bool nope = dc < kNope / 8;
    o0 = nope ? 8 * dc : 16 * dc - kNope;
    o1 = nope ? 576 + 8 * (dc >> 4) : 16 * dc - kNope + 8;
  }
  RawChunk r;
  if constexpr (NTG) {
    r.lo = __builtin_nontemporal_load((gv2u)(rp + o0));
    r.hi = __builtin_nontemporal_load((gv2u)(rp + o1));
  } else {
    r.lo = *(gv2u)(rp + o0);
    r.hi = *(gv2u)(rp + o1);
  }
  return r;
}

// Raw chunk -> 8 bf16 (4 dwords).  Branch-free: the FP8 conversion is always computed and selected
// per lane (nope lanes of FP8 rows take it; rope lanes and BF16 rows keep the raw bits).
template <int WF, int CF>
__device__ __forceinline__ uint4 raw_to_bf16(const RawChunk& r, uint64_t code, int dc) {
  uint4 w = make_uint4(r.lo[0], r.lo[1], r.hi[0], r.hi[1]);
  if constexpr (WF == kRowFP8 || CF == kRowFP8) {
    const int fmt = (code & kCodeComp) ? CF : WF;
    const bool fp8_lane = fmt == kRowFP8 && dc < kNope / 8;
    float v[8];
    fp8x4_to_f32(r.lo[0], v);
    fp8x4_to_f32(r.lo[1], v + 4);
    const float sc = __uint_as_float((dc >> 3) & 1 ? r.hi[1] : r.hi[0]);
    const uint32_t c0 = pack_bf16x2(v[0] * sc, v[1] * sc), c1 = pack_bf16x2(v[2] * sc, v[3] * sc);
    const uint32_t c2 = pack_bf16x2(v[4] * sc, v[5] * sc), c3 = pack_bf16x2(v[6] * sc, v[7] * sc);
    w.x = fp8_lane ? c0 : w.x;
    w.y = fp8_lane ? c1 : w.y;
    w.z = fp8_lane ? c2 : w.z;
    w.w = fp8_lane ? c3 : w.w;
  }
  return w;
}

// Row gathers shared by both roles of the 64-head kernel: a wave owns rows rb .. rb+3 of every
// 32-slot tile of its block's range, entry 4t + i = row rb + i of tile t.  Their codes are resolved
// into VGPRs (lane l of word j holds entry 64j + l: two words cover the 32 tiles of a block), and
// the wave's nibble of each tile's valid-slot mask goes to byte `vm_slot` of that tile's 8 mask
// bytes in LDS.
__device__ __forceinline__ void gather_codes(const AttnArgs& a, int q, int r, int s_begin, int nt, int n_idx,
                                             int rb, int lane, uint32_t* cw_lo, uint32_t* cw_hi, uint8_t* vm8,
                                             int vm_slot, const int32_t* idx_list = nullptr,
                                             const int32_t* rows_list = nullptr) {
  int sl[4];
  bool in[4], ok[4];
  uint64_t c[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = 64 * j + lane;                   // entry: tile e / 4, row e % 4
    sl[j] = s_begin + (e >> 2) * kTile + rb + (e & 3);
    in[j] = j < 2 && e < 4 * nt && sl[j] < n_idx;
  }
  slot_codes4(a, q, r, sl, in, c, ok, idx_list, rows_list);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    cw_lo[j] = (uint32_t)c[j];
    cw_hi[j] = (uint32_t)(c[j] >> 32);
    const uint64_t bal = __ballot(ok[j]);
    const int t = 16 * j + lane;                   // lanes 0..15 write the nibbles of tiles 16j .. 16j+15
    if (lane < 16 && t < nt) vm8[8 * t + vm_slot] = (uint8_t)((bal >> (4 * lane)) & 0xFu);
  }
}

// Issue the loads of the wave's four rows of tile k (codes picked from VGPRs with lane reads).
template <int WF, int CF, bool NTG>
__device__ __forceinline__ void gather_fetch(int k, const uint32_t* cw_lo, const uint32_t* cw_hi, int lane,
                                             RawChunk* rw, uint64_t* c4) {
  const uint32_t lo = (k >> 4) ? cw_lo[1] : cw_lo[0], hi = (k >> 4) ? cw_hi[1] : cw_hi[0];
  const int l0 = (4 * k) & 63;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    c4[i] = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane(hi, l0 + i) << 32) |
            (uint32_t)__builtin_amdgcn_readlane(lo, l0 + i);   // zero-extended: the lane read is an int
#pragma unroll
  for (int i = 0; i < 4; ++i) rw[i] = load_raw<WF, CF, NTG>(c4[i], lane);
}

// Write the wave's four rows of a tile into the LDS tile K (dequantised to bf16).
template <int WF, int CF>
__device__ __forceinline__ void gather_stage(uint16_t* K, int rb, const RawChunk* rw, const uint64_t* c4, int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i) *(uint4*)&K[(rb + i) * kKrStride + 8 * lane] = raw_to_bf16<WF, CF>(rw[i], c4[i], lane);
}


// Tiles of a block's range.  A causal prefill's lists end with invalid slots past the visible
// prefix (the selection pads with -1 when fewer than k entries are visible, and dense lists stop
// at the visible count), so an unsplit block stops after the last tile that can hold a valid
// slot: n_win + min(n_comp, (t + 1) / ratio) slots for the query at position t.  Early prefill
// positions see few entries, so this skips about a tenth of the 8,192-query prefill's tiles.
__device__ __forceinline__ int attn_block_tiles(const AttnArgs& a, int q, int n_tiles, int t_begin, int tps) {
  int nt = max(0, min(n_tiles, t_begin + tps) - t_begin);
  if (a.trim_ratio > 0 && a.req_mode == 2 && a.n_split == 1) {
    const int64_t vis = (a.pos0 + q + 1) / a.trim_ratio;
    const int64_t n_eff = a.n_win + (vis < a.n_comp ? vis : a.n_comp);
    nt = min(nt, (int)((n_eff + kTile - 1) / kTile));
  }
  return nt;
}

constexpr int kAttnThreads = 512;   // waves 0-3 consume (matrix cores), waves 4-7 produce (gathers)
#ifndef CSA_ATTN_DEPTH
#define CSA_ATTN_DEPTH 4
#endif
constexpr int kDepth = CSA_ATTN_DEPTH;   // tiles of row gathers in flight per producer wave
#ifndef CSA_SCORE_DEPTH
#define CSA_SCORE_DEPTH 2
#endif
constexpr int kScoreDepth = CSA_SCORE_DEPTH;   // the same for the score waves of the 64-head kernel

// Producer side of the matrix-core kernels (waves 4-7 of a block): wave 4+p gathers rows 8p ..
// 8p+7 of every 32-slot tile, one 16-B chunk (8 dims) per lane, kDepth tiles ahead in registers,
// and dequantises tile j into ring buffer j % 3 just before barrier j, for j < nt.  The consumers
// read tile j after barrier j and are done with it before barrier j + 2, so the buffer is free
// again when tile j + 3 is staged.  The producers pass `nbar` >= nt + 1 barriers in all.
template <int WF, int CF, bool NTG>
__device__ __forceinline__ void produce_tiles(const uint64_t* codes, uint16_t (*Kr)[kTile * kKrStride], int nt,
                                              int nbar, int lane, int wave) {
  const int pw = wave - 4;
  RawChunk raw[kDepth][8];
  uint64_t rc[kDepth][8];
  auto fetch = [&](int k, RawChunk* rw, uint64_t* c8) {
    const int base = k * kTile + 8 * pw;
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      const uint4 c = *(const uint4*)&codes[base + i];
      c8[i] = ((uint64_t)__builtin_amdgcn_readfirstlane(c.y) << 32) | (uint32_t)__builtin_amdgcn_readfirstlane(c.x);
      c8[i + 1] = ((uint64_t)__builtin_amdgcn_readfirstlane(c.w) << 32) | (uint32_t)__builtin_amdgcn_readfirstlane(c.z);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) rw[i] = load_raw<WF, CF, NTG>(c8[i], lane);
  };
  auto stage = [&](int buf, const RawChunk* rw, const uint64_t* c8) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      *(uint4*)&Kr[buf][(8 * pw + i) * kKrStride + 8 * lane] = raw_to_bf16<WF, CF>(rw[i], c8[i], lane);
  };
  // tile j lives in raw slot j % kDepth from its fetch until it is staged
#pragma unroll
  for (int j = 0; j < kDepth; ++j)
    if (j < nt) fetch(j, raw[j], rc[j]);
  if (nt > 0) {
    stage(0, raw[0], rc[0]);
    if (kDepth < nt) fetch(kDepth, raw[0], rc[0]);
  }
  __syncthreads();
  int buf = 1;   // (k + 1) % 3
  for (int k = 0; k < nt; k += kDepth) {
#pragma unroll
    for (int u = 0; u < kDepth; ++u) {
      if (k + u < nt) {
        constexpr int kDepthC = kDepth;
        const int sl = (u + 1) % kDepthC;
        if (k + u + 1 < nt) {
          stage(buf, raw[sl], rc[sl]);
          if (k + u + 1 + kDepth < nt) fetch(k + u + 1 + kDepth, raw[sl], rc[sl]);
        }
        buf = buf == 2 ? 0 : buf + 1;
        __syncthreads();
      }
    }
  }
  for (int j = nt + 1; j < nbar; ++j) __syncthreads();
}

// Selection inside the attention blocks (SEL): every block of a query first selects the query's
// k rows itself, exactly as topk_single_kernel does (its block_threshold / block_emit with this
// block's 512 threads, PER entries each), into LDS borrowed from tile slots 1-3 of the ring (no
// tile is staged there before the first barrier of the tile loop).  Its slot codes then come from
// LDS: the step saves the selection launch and the global round trip of the index list.  The
// blocks of split 0 also write the index list and rows for the caller.
constexpr int kSelPer = 32;                                           // entries per thread
constexpr int kSelRowMax = kAttnThreads * kSelPer;                    // 16,384 entries
constexpr int kSelOff = kTile * kKrStride * 2;                        // byte offset: tile slot 1
constexpr int kSelListOff = kSelOff + 32768;                          // after SelShared (< 32 KB)
constexpr int kSelRowsOff = kSelListOff + 4 * kMaxSlots;
constexpr int kSelPtOff = kSelRowsOff + 4 * kMaxSlots;
static_assert(sizeof(SelShared<kAttnThreads>) <= 32768, "selection LDS fits its space");
constexpr int kSelSketchPer = 8;                                      // sketch entries per thread
static_assert(kSelPtOff + 4 * (kSelRowMax / kPage) <= 3 * kTile * kKrStride * 2, "selection LDS fits the 16-head ring");
static_assert(kSelPtOff + 4 * (kSelRowMax / kPage) <= 4 * kTile * kKrStride * 2, "selection LDS fits the ring");

// Visible entries and tokens seen of a decode query that is its request's only query, from the
// request's context length: row_extent for win_mode 1 with q_per_req 1, without its branches and
// divisions (the prologue's scalar instructions are issued by every wave of the block).
__device__ __forceinline__ int64_t decode1_extent(const TopkArgs& t, int32_t ctx, int64_t& seen) {
  seen = ctx < 0 ? 0 : (ctx > t.max_ctx ? t.max_ctx : (int64_t)ctx);
  const int64_t nv = seen / 4;
  return nv > t.max_n_vis ? t.max_n_vis : nv;
}

// Selects query q's rows into LDS: idx_list[0 .. n_win + k) (the ring window, then the k entries in
// ascending order, -1 past the visible ones) and rows_list[0 .. k) (their pool rows, -1 if none).
// Every load of the prologue (the context length, the first page ids, the scores up to the widest
// row, all in bounds and masked once the row's length is known) is issued before the first wait: a
// chain of dependent loads (length, then page ids, then scores) cost several memory round trips per
// block.  issue_more() issues the caller's own loads after the first barrier, where nothing waits
// for them until the selection is done (issued earlier, the waits for the scores would also wait for
// them: the load counter drains in order).
template <class IssueMore>
__device__ __forceinline__ void select_rows(const TopkArgs& t, int q, uint8_t* lds, bool write_out, IssueMore issue_more) {
  const int tid = threadIdx.x;
  SelShared<kAttnThreads>& sh = *(SelShared<kAttnThreads>*)(lds + kSelOff);
  int32_t* idx_list = (int32_t*)(lds + kSelListOff);
  int32_t* rows_list = (int32_t*)(lds + kSelRowsOff);
  int32_t* pt_lds = (int32_t*)(lds + kSelPtOff);
  const int k = t.k;
  const int32_t ctx = t.ctx_len[q];   // decode, one query per request (attn_select_fused)
  const int32_t* pt = t.page_table + (int64_t)q * t.max_pages;
  const int n_pt = t.max_pages < kSelRowMax / kPage ? t.max_pages : kSelRowMax / kPage;
  const int32_t pg_mine = tid < n_pt ? pt[tid] : -1;
  const float* row = t.logits + (int64_t)q * t.ld;
  const int c0 = tid * kSelPer;
  float v[kSelPer];
#pragma unroll
  for (int j = 0; j < kSelPer; j += 4) {
    const int c = c0 + j;
    const float4 x = *(const float4*)(row + (c < t.max_n_vis ? c : 0));   // ld >= max_n_vis, ld % 4 == 0
    v[j] = x.x; v[j + 1] = x.y; v[j + 2] = x.z; v[j + 3] = x.w;
  }
  int64_t seen;
  const int64_t nv = decode1_extent(t, ctx, seen);
  auto row_of = [&](int c, int pg) { return (unsigned)pg < (unsigned)t.num_pages ? pg * kPage + (c & (kPage - 1)) : -1; };
  if (tid < kWin) {
    const int64_t p = seen - kWin + tid;
    idx_list[tid] = p >= 0 ? ring_slot(p, t.ring) : -1;
  }
  if (tid < n_pt) pt_lds[tid] = pg_mine;
  uint32_t key[kSelPer];
  uint32_t vm = 0;
  if (nv > k) {
    for (int i = tid; i < kHistBins; i += kAttnThreads) sh.bins[i] = 0u;
    if (tid == 0) sh.s_ncand = 0u;
#pragma unroll
    for (int j = 0; j < kSelPer; ++j) key[j] = order_key_raw(v[j]);
    vm = prefix_mask<kSelPer>(c0, nv);
    publish_extremes<kAttnThreads, kSelPer>(key, vm, sh);   // read after the barrier below
  }
  __syncthreads();
  issue_more();
  if (nv <= k) {
    for (int i = tid; i < k; i += kAttnThreads) {
      idx_list[kWin + i] = i < nv ? i : -1;
      rows_list[i] = i < nv ? row_of(i, pt_lds[i >> 6]) : -1;
    }
  } else {
    block_threshold<kAttnThreads, kSelPer, true, true>(key, vm, (uint32_t)k, sh);
    block_emit<kAttnThreads, kSelPer>(key, vm, sh.s_T, sh.s_need, (uint32_t)k, [&](int j) { return c0 + j; }, sh);
    const int32_t* sel = (const int32_t*)sh.cand_sel;
    for (int i = tid; i < k; i += kAttnThreads) {
      const int c = sel[i];
      const int rw = row_of(c, pt_lds[c >> 6]);
      CSA_DBG_COUNT(rw < 0);   // a selected entry on a page with no page id in the pool
      idx_list[kWin + i] = c;
      rows_list[i] = rw;
    }
  }
  __syncthreads();
  if (write_out) {
    for (int i = tid; i < kWin + k; i += kAttnThreads) t.idx[(int64_t)q * t.ld_idx - kWin + i] = idx_list[i];
    for (int i = tid; i < k; i += kAttnThreads) t.rows[(int64_t)q * t.ld_rows + i] = rows_list[i];
  }
}

// The same for long decode rows, from the indexer's per-wave sketches as topk_sketch_kernel
// selects them (PER sketch entries per thread): the sketches' exact k-th largest key T decides the
// row when every wave's bound lies below T; otherwise the block rescores the row if it has no
// stored scores and selects from the full row (select_streamed), writing straight into the lists.
// The sketch entries and wave bounds are loaded with the context length, up to the widest row (in
// bounds, masked once the row's length is known), before the first wait; issue_more() comes after
// the first barrier (after the selection's own waits).
template <int PER, class IssueMore>
__device__ __forceinline__ void select_rows_sketch(const TopkArgs& t, int q, uint8_t* lds, bool write_out,
                                                   IssueMore issue_more) {
  constexpr int NT = kAttnThreads;
  const int tid = threadIdx.x;
  SelShared<NT>& sh = *(SelShared<NT>*)(lds + kSelOff);
  int32_t* idx_list = (int32_t*)(lds + kSelListOff);
  int32_t* rows_list = (int32_t*)(lds + kSelRowsOff);
  const int k = t.k;
  const int32_t ctx = t.ctx_len[q];   // decode, one query per request (attn_select_fused)
  const uint2* top = t.sk_top + (int64_t)q * t.sk_waves * kSketchTop;
  const uint32_t* bound = t.sk_bound + (int64_t)q * t.sk_waves;
  const int64_t n_u_max = (int64_t)t.sk_waves * kSketchTop;
  uint32_t key[PER], idx[PER];
  const int64_t u0 = (int64_t)tid * PER;
#pragma unroll
  for (int j = 0; j < PER; j += 2) {
    const int64_t u = u0 + j;
    const uint4 x = *(const uint4*)&top[u < n_u_max ? u : 0];
    key[j] = x.x; idx[j] = x.y; key[j + 1] = x.z; idx[j + 1] = x.w;
  }
  constexpr int kBnd = (kSketchMaxWaves + NT - 1) / NT;
  uint32_t bnd[kBnd];
#pragma unroll
  for (int i = 0; i < kBnd; ++i) {
    const int64_t W = tid + (int64_t)i * NT;
    bnd[i] = W < t.sk_waves ? bound[W] : 0u;
  }
  int64_t seen;
  const int64_t nv = decode1_extent(t, ctx, seen);
  const int32_t* pt = t.page_table + (int64_t)q * t.max_pages;
  auto row_of = [&](int c) {
    const int pg = pt[c >> 6];
    return (unsigned)pg < (unsigned)t.num_pages ? pg * kPage + (c & (kPage - 1)) : -1;
  };
  if (tid < kWin) {
    const int64_t p = seen - kWin + tid;
    idx_list[tid] = p >= 0 ? ring_slot(p, t.ring) : -1;
  }
  const int64_t n_w = (nv + kSketchSpan - 1) / kSketchSpan;
  const int64_t n_u = n_w * kSketchTop;
  uint32_t vm = 0u;
  if (nv > k) {
#pragma unroll
    for (int i = 0; i < kBnd; ++i) bnd[i] = tid + (int64_t)i * NT < n_w ? bnd[i] : 0u;
    for (int i = tid; i < kHistBins; i += NT) sh.bins[i] = 0u;
    if (tid == 0) sh.s_ncand = 0u;
#pragma unroll
    for (int j = 0; j < PER; ++j) vm |= (u0 + j < n_u && idx[j] != 0xFFFFFFFFu ? 1u : 0u) << j;
    const uint32_t wsum = wave_inclusive_scan(__popc(vm));
    if ((tid & 63) == 63) sh.scan[tid >> 6] = wsum;
  }
  __syncthreads();
  issue_more();
  if (nv <= k) {   // block-uniform
    for (int i = tid; i < k; i += NT) {
      idx_list[kWin + i] = i < nv ? i : -1;
      rows_list[i] = i < nv ? row_of(i) : -1;
    }
  } else {
    uint32_t n_real = 0u;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) n_real += sh.scan[w];
    bool from_sketch = n_real >= (uint32_t)k;
    if (from_sketch) {
      block_threshold<NT, PER>(key, vm, (uint32_t)k, sh);
      const uint32_t T = sh.s_T;
      bool reach = false;
#pragma unroll
      for (int i = 0; i < kBnd; ++i) reach |= tid + (int64_t)i * NT < n_w && bnd[i] >= T;
      from_sketch = !__syncthreads_or(reach);
    }
    if (from_sketch) {
      block_emit<NT, PER>(key, vm, sh.s_T, sh.s_need, (uint32_t)k, [&](int j) { return (int32_t)idx[j]; }, sh);
      const int32_t* sel = (const int32_t*)sh.cand_sel;
      for (int i = tid; i < k; i += NT) {
        const int c = sel[i];
        const int rw = row_of(c);
        CSA_DBG_COUNT(rw < 0);
        idx_list[kWin + i] = c;
        rows_list[i] = rw;
      }
    } else {
      if (t.ia.sk_rescore_from > 0 && nv >= t.ia.sk_rescore_from) {
        // the indexer stored no scores for this row: rescore it, each wave a span at a time (every
        // block of the query writes the same scores; each reads back only its own)
        const int wave = tid >> 6, lane = tid & 63;
        const int nhg = (t.ia.HI + 15) / 16;
        for (int64_t W = wave; W < n_w; W += NT / 64) {
          if (t.ia.dt == 3) {
            switch (nhg) {
              case 1: rescore_span<1, true>(t.ia, q, W, lane); break;
              case 2: rescore_span<2, true>(t.ia, q, W, lane); break;
              case 3: rescore_span<3, true>(t.ia, q, W, lane); break;
              default: rescore_span<4, true>(t.ia, q, W, lane); break;
            }
          } else {
            switch (nhg) {
              case 1: rescore_span<1, false>(t.ia, q, W, lane); break;
              case 2: rescore_span<2, false>(t.ia, q, W, lane); break;
              case 3: rescore_span<3, false>(t.ia, q, W, lane); break;
              default: rescore_span<4, false>(t.ia, q, W, lane); break;
            }
          }
        }
        __syncthreads();   // the block reads the rescored row next (workgroup scope: one L1)
      }
      select_streamed<NT>(t, q, nv, (uint32_t)k, sh, idx_list + kWin, rows_list, pt);
    }
  }
  __syncthreads();
  if (write_out) {
    for (int i = tid; i < kWin + k; i += NT) t.idx[(int64_t)q * t.ld_idx - kWin + i] = idx_list[i];
    for (int i = tid; i < k; i += NT) t.rows[(int64_t)q * t.ld_rows + i] = rows_list[i];
  }
}

template <int WF, int CF, bool NTG, bool SEL = false>
__global__ __launch_bounds__(kAttnThreads, 1) void attn_bf16_kernel(AttnArgs a, TopkArgs t) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
  // grid (query, head block, split): queries vary fastest in the dispatch order, so with Q a
  // multiple of 8 every split of a query (and the combine blocks that read its partials) runs on the
  // same XCD and shares its L2
  const int q = blockIdx.x, split = blockIdx.z;
  const int Hpad = (a.H + 15) & ~15;
  const int h_base = blockIdx.y * 64;

  __shared__ __align__(16) uint16_t Kr[4][kTile * kKrStride];   // ring of four bf16 row tiles
  __shared__ __align__(16) uint4 Ps[2][4][64];                   // P^T operand of each head group
  __shared__ __align__(16) v4f Sx[2][4][2][64];                  // partial scores for the partner wave
  __shared__ __align__(16) int Fl[2][4];                         // head group rescaled this tile
  __shared__ float As[2][64];                                    // its per-head rescale factors
  __shared__ float Ms[64], Ls[64], Xs[4][64];
  // valid slots of each tile: byte w holds rows 8w .. 8w+3 (score wave w), byte 4 + w rows
  // 8w+4 .. 8w+7 (value wave w), one bit per row in the low nibble
  __shared__ __align__(8) uint8_t vm8[kMaxSlots / kTile][8];

  const int n_idx = a.n_win + a.n_comp;
  const int n_tiles = (n_idx + kTile - 1) / kTile;
  const int tps = a.tiles_per_split;
  const int t_begin = split * tps;
  const int nt = attn_block_tiles(a, q, n_tiles, t_begin, tps);   // tiles of this block
  // the fused selection runs only for decode with one query per request (attn_select_fused)
  const int r = SEL ? q : (a.req_mode == 1 ? q / a.q_per_req : (a.req_mode == 2 ? 0 : a.q_req[q]));
  const int s_begin = t_begin * kTile;
  const int32_t* idx_list = nullptr;
  const int32_t* rows_list = nullptr;
  // score waves: wave w computes the scores of head groups w and w ^ 1 over dims [256 (w & 1),
  // +256), so every K fragment it reads feeds two MFMAs and each K element is read by two waves
  // instead of four; the partial scores of head group w ^ 1 go to wave w ^ 1 through LDS.  q stays
  // in registers as the QK B operand: qo[ks] / qx[ks] hold dims 256 (w & 1) + 32ks + 8g .. +7 of
  // head n of group w / w ^ 1.  Padded heads read head 0's row; their results are never written.
  v8bf qo[8], qx[8];
  auto load_q = [&] {
    const int ho = h_base + 16 * wave + n, hx = h_base + 16 * (wave ^ 1) + n;
    const int d0 = 256 * (wave & 1) + 8 * g;
    const uint16_t* qpo = (const uint16_t*)a.q + ((int64_t)q * a.H + (ho < a.H ? ho : 0)) * kD + d0;
    const uint16_t* qpx = (const uint16_t*)a.q + ((int64_t)q * a.H + (hx < a.H ? hx : 0)) * kD + d0;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      qo[ks] = *(const v8bf*)(qpo + 32 * ks);
      qx[ks] = *(const v8bf*)(qpx + 32 * ks);
    }
  };
  if constexpr (SEL) {
    // q does not depend on the selection: its loads, issued behind the selection's, overlap it
    uint8_t* lds = (uint8_t*)&Kr[0][0];
    select_rows(t, q, lds, split == 0 && blockIdx.y == 0, [&] {
      if (wave < 4) load_q();
    });
    idx_list = (const int32_t*)(lds + kSelListOff);
    rows_list = (const int32_t*)(lds + kSelRowsOff);
  }

  float m = kNegBig, lsum = 0.f;   // score-wave softmax state of head h_base + 16 wave + n
  v4f acc[4][8];                   // value waves: O^T[128 dw + 16 dt + 4 g + i][h_base + 16 hg + n]
#pragma unroll
  for (int hg = 0; hg < 4; ++hg)
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) acc[hg][dt] = v4f{0.f, 0.f, 0.f, 0.f};

  // Phase p (ending at barrier p) of the tile loop: the score waves issue the scores of tile p on
  // the matrix cores, run the softmax of tile p - 1 (its scores were computed in phase p - 1) and
  // publish its P^T, then stage tile p + 1 into the ring slot of tile p - 3, which nobody reads
  // after phase p - 1; the value waves accumulate P.V of tile p - 2.
  if (wave < 4) {
    const int rb = 8 * wave;   // gathered rows rb .. rb+3 of every tile
    uint32_t cw_lo[2], cw_hi[2];
    gather_codes(a, q, r, s_begin, nt, n_idx, rb, lane, cw_lo, cw_hi, &vm8[0][0], wave, idx_list, rows_list);
    // q after the codes: the codes' index loads then do not wait behind the 32 q loads
    if constexpr (!SEL) load_q();
    RawChunk raw[kScoreDepth][4];
    uint64_t rc[kScoreDepth][4];
    auto fetch = [&](int t, RawChunk* rw, uint64_t* c4) { gather_fetch<WF, CF, NTG>(t, cw_lo, cw_hi, lane, rw, c4); };
    auto stage = [&](uint16_t* K, const RawChunk* rw, const uint64_t* c4) { gather_stage<WF, CF>(K, rb, rw, c4, lane); };
    // partial S^T[key][head] over this wave's 256 dims for keys 0..15 ([0]) and 16..31 ([1]), of
    // head group w (so) and w ^ 1 (sx)
    const int dk = 256 * (wave & 1);
    auto scores = [&](const uint16_t* K, v4f* so, v4f* sx) {
      v4f o0 = v4f{0.f, 0.f, 0.f, 0.f}, o1 = o0, x0 = o0, x1 = o0;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const v8bf k0 = *(const v8bf*)&K[n * kKrStride + dk + 32 * ks + 8 * g];
        const v8bf k1 = *(const v8bf*)&K[(16 + n) * kKrStride + dk + 32 * ks + 8 * g];
        o0 = mma_bf16(k0, qo[ks], o0);
        x0 = mma_bf16(k0, qx[ks], x0);
        o1 = mma_bf16(k1, qo[ks], o1);
        x1 = mma_bf16(k1, qx[ks], x1);
      }
      so[0] = o0;
      so[1] = o1;
      sx[0] = x0;
      sx[1] = x1;
    };
    const float sc = a.softmax_scale * kLog2e;
    // softmax of tile t with valid-slot mask vm (vm = 0: no slot, the state is left unchanged); the
    // scores are this wave's partial plus the partner's, published at the end of the previous phase
    auto softmax = [&](int t, uint32_t vm, const v4f* sv, const v4f& y0, const v4f& y1) {
      const int pb = t & 1;
      float x[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[i] = (vm >> (4 * g + i)) & 1u ? (sv[0][i] + y0[i]) * sc : -INFINITY;
        x[4 + i] = (vm >> (16 + 4 * g + i)) & 1u ? (sv[1][i] + y1[i]) * sc : -INFINITY;
      }
      float tmax = x[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) tmax = fmaxf(tmax, x[e]);
      tmax = row_group_max(tmax);
      // lazy rescaling: the reference max moves only when a head's max grows by more than 2^8, so
      // the value waves rescale their accumulators rarely; p = 2^(S - m) then stays below 256.  The
      // update is branch-free here (alpha = 1 when the max stays), so the whole softmax is one basic
      // block that the compiler can interleave with the matrix-core work of the next tile.
      const bool grow = tmax > m + kRescaleLog2;
      const float m_new = grow ? tmax : m;
      const float alpha = __builtin_amdgcn_exp2f(m - m_new);
      lsum *= alpha;
      m = m_new;
      const int fl = __ballot(grow) != 0ull;
      float pr[8], psum = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pr[e] = __builtin_amdgcn_exp2f(x[e] - m);
        psum += pr[e];
      }
      lsum += psum;
      // slot 8g+4mt+i of the K step <-> key 16mt+4g+i: these 8 values are exactly this lane's part
      // of the P^T operand, for every value wave
      Ps[pb][wave][lane] = make_uint4(pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3]),
                                      pack_bf16x2(pr[4], pr[5]), pack_bf16x2(pr[6], pr[7]));
      if (g == 0) As[pb][16 * wave + n] = alpha;
      if (lane == 0) Fl[pb][wave] = fl;
    };
    // tile j lives in raw slot j % kScoreDepth from its fetch until it is staged
#pragma unroll
    for (int j = 0; j < kScoreDepth; ++j)
      if (j < nt) fetch(j, raw[j], rc[j]);
    if (nt > 0) {
      stage(Kr[0], raw[0], rc[0]);
      if (kScoreDepth < nt) fetch(kScoreDepth, raw[0], rc[0]);
    }
    __syncthreads();
    v4f sv[2][2];   // own partial scores of the tiles of even and odd index
    for (int p0 = 0; p0 <= nt; p0 += kScoreDepth) {
#pragma unroll
      for (int u = 0; u < kScoreDepth; ++u) {
        const int p = p0 + u;
        if (p <= nt) {
          constexpr int kDepthC = kScoreDepth;
          const int sl = (u + 1) % kDepthC;   // raw slot of tile p + 1
          // p = nt scores a stale tile (never used); p = 0 runs a softmax over no slot (a no-op)
          // the partner's partial scores of tile p - 1 (published before the last barrier), read
          // before this tile's operands so their latency hides behind the matrix-core work
          const v4f y0 = Sx[(p - 1) & 1][wave ^ 1][0][lane], y1 = Sx[(p - 1) & 1][wave ^ 1][1][lane];
          v4f sxp[2];
          scores(Kr[p & 3], sv[u & 1], sxp);
          uint32_t vm = 0u;
          if (p >= 1) {
            const uint2 mb = *(const uint2*)&vm8[p - 1][0];
            vm = mb.x | (mb.y << 4);
          }
          softmax(p - 1, vm, sv[(u + 1) & 1], y0, y1);
          // the partner's partial scores of tile p, read by it in the next phase (tile p + 2 reuses
          // the buffer after the barrier that follows that read)
          Sx[p & 1][wave][0][lane] = sxp[0];
          Sx[p & 1][wave][1][lane] = sxp[1];
          // staging last keeps its LDS writes out of the way of this phase's operand reads
          if (p + 1 < nt) {
            stage(Kr[(p + 1) & 3], raw[sl], rc[sl]);
            if (p + 1 + kScoreDepth < nt) fetch(p + 1 + kScoreDepth, raw[sl], rc[sl]);
          }
          __syncthreads();
        }
      }
    }
    __syncthreads();   // phase nt + 1: the value waves finish tile nt - 1
    const float ltot = row_group_sum(lsum);
    if (g == 0) {
      Ms[16 * wave + n] = m;
      Ls[16 * wave + n] = ltot;
    }
  } else {
    const int dw = wave - 4;   // output dims [128 dw, 128 dw + 128)
    const int rb = 8 * dw + 4;   // gathered rows rb .. rb+3 of every tile
    uint32_t cw_lo[2], cw_hi[2];
    gather_codes(a, q, r, s_begin, nt, n_idx, rb, lane, cw_lo, cw_hi, &vm8[0][0], 4 + dw, idx_list, rows_list);
    // one tile of gathers in flight: the value waves' own work is the shorter of the two roles, so
    // they can wait for a gather without lengthening the phase
    RawChunk raw[4];
    uint64_t rc[4];
    if (nt > 0) {
      gather_fetch<WF, CF, NTG>(0, cw_lo, cw_hi, lane, raw, rc);
      gather_stage<WF, CF>(Kr[0], rb, raw, rc, lane);
      if (nt > 1) gather_fetch<WF, CF, NTG>(1, cw_lo, cw_hi, lane, raw, rc);
    }
    __syncthreads();
    for (int p = 0; p <= nt + 1; ++p) {
      // staging first: its VALU work and waits overlap the score waves' matrix-core burst at the
      // start of the phase, and P.V then runs while the score waves do their softmax
      if (p + 1 < nt) {
        gather_stage<WF, CF>(Kr[(p + 1) & 3], rb, raw, rc, lane);
        if (p + 2 < nt) gather_fetch<WF, CF, NTG>(p + 2, cw_lo, cw_hi, lane, raw, rc);
      }
      if (p >= 2) {
        const int t = p - 2;
        const int pb = t & 1;
        const uint16_t* K = Kr[t & 3];
        const int4 f4 = *(const int4*)Fl[pb];
        if (__builtin_expect((f4.x | f4.y | f4.z | f4.w) != 0, 0)) {
          __asm__ volatile("" ::: "memory");
#pragma unroll
          for (int hg = 0; hg < 4; ++hg) {
            const float al = As[pb][16 * hg + n];
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) acc[hg][dt] *= al;
          }
        }
        v8bf pf[4];
#pragma unroll
        for (int hg = 0; hg < 4; ++hg) pf[hg] = __builtin_bit_cast(v8bf, Ps[pb][hg][lane]);
        // O^T[d][head] += V^T[d][slot] . P^T[slot][head] over this wave's 128 dims, all head
        // groups; V^T comes from the row-major tile through the transposing LDS read: source lane s
        // of group g points at key row 4g + s/4 (slots 8g..8g+3) or 16 + 4g + s/4 (slots
        // 8g+4..8g+7), dims 4(s%4) .. +3
        const uint16_t* tr_lo = &K[(4 * g + (n >> 2)) * kKrStride + 4 * (n & 3) + 128 * dw];
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          const v4s lo = lds_read_tr16(tr_lo + 16 * dt);
          const v4s hi = lds_read_tr16(tr_lo + 16 * kKrStride + 16 * dt);
          const v8bf vv = __builtin_bit_cast(v8bf, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
          for (int hg = 0; hg < 4; ++hg) acc[hg][dt] = mma_bf16(vv, pf[hg], acc[hg][dt]);
        }
      }
      __syncthreads();
    }
  }
  __syncthreads();
  const int dw = wave - 4;   // value waves: output dims [128 dw, 128 dw + 128)
  const int dbase = 128 * dw + 4 * g;
  // 16-bit output rows (bf16 results, fp16 partials) are staged in the idle row tiles, 1056 B per
  // head, so that every wave then stores whole 1 KB rows with one instruction each
  constexpr int kStage = kKrStride;
  uint16_t* stg = &Kr[0][0];
  static_assert(64 * kStage <= 4 * kTile * kKrStride, "staging fits the row tiles");
  auto store_rows = [&](uint16_t* base, int64_t row_stride, int nrows) {
    // wave w writes staged rows 8w .. 8w+7 (those below nrows) to base + row * row_stride
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int rr = 8 * wave + i;
      if (rr < nrows) *(uint4*)(base + rr * row_stride + 8 * lane) = *(const uint4*)&stg[rr * kStage + 8 * lane];
    }
  };
  if (a.n_split == 1) {
    if (wave >= 4) {
      float inv[4];
#pragma unroll
      for (int hg = 0; hg < 4; ++hg) {
        const int h = h_base + 16 * hg + n;
        const float mh = Ms[16 * hg + n], lh = Ls[16 * hg + n];
        const float sk = a.sink[h < a.H ? h : 0] * kLog2e;
        const float M = fmaxf(mh, sk);
        const float f = exp2f(mh - M);
        inv[hg] = f / (lh * f + exp2f(sk - M));
      }
      if (a.out_dt == 0) {
#pragma unroll
        for (int hg = 0; hg < 4; ++hg) {
          const int h = h_base + 16 * hg + n;
          if (h >= a.H) continue;
          const int64_t ob = ((int64_t)q * a.H + h) * kD + dbase;
#pragma unroll
          for (int dt = 0; dt < 8; ++dt)
            store4(a.out, 0, ob + 16 * dt, acc[hg][dt][0] * inv[hg], acc[hg][dt][1] * inv[hg],
                   acc[hg][dt][2] * inv[hg], acc[hg][dt][3] * inv[hg]);
        }
      } else {
#pragma unroll
        for (int hg = 0; hg < 4; ++hg)
#pragma unroll
          for (int dt = 0; dt < 8; ++dt)
            *(uint2*)&stg[(16 * hg + n) * kStage + dbase + 16 * dt] =
                make_uint2(pack_bf16x2(acc[hg][dt][0] * inv[hg], acc[hg][dt][1] * inv[hg]),
                           pack_bf16x2(acc[hg][dt][2] * inv[hg], acc[hg][dt][3] * inv[hg]));
      }
    }
    if (a.out_dt == 0) return;
    __syncthreads();
    store_rows((uint16_t*)a.out + ((int64_t)q * a.H + h_base) * kD, kD, min(64, a.H - h_base));
    return;
  }
  // split-K partial of each head: m, l, amax = max |acc| over the 512 dims (fp32) and acc / amax
  // as fp16 (|value| <= 1, so the only loss is fp16's 11-bit rounding relative to amax)
  if (wave >= 4) {
#pragma unroll
    for (int hg = 0; hg < 4; ++hg) {
      float mx = 0.f;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, fabsf(acc[hg][dt][i]));
      mx = row_group_max(mx);
      if (g == 0) Xs[dw][16 * hg + n] = mx;
    }
  }
  __syncthreads();
  const int64_t prow0 = ((int64_t)q * a.n_split + split) * Hpad + h_base;   // partial row of head h_base
  if (wave >= 4) {
    float* pml = (float*)((uint8_t*)a.part + (size_t)a.Q * a.n_split * Hpad * kD * sizeof(uint16_t));
#pragma unroll
    for (int hg = 0; hg < 4; ++hg) {
      const int hl = 16 * hg + n;
      const float amax = fmaxf(fmaxf(Xs[0][hl], Xs[1][hl]), fmaxf(Xs[2][hl], Xs[3][hl]));
      const float f = amax > 0.f ? 1.f / amax : 0.f;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        *(uint2*)&stg[hl * kStage + dbase + 16 * dt] = make_uint2(pack_f16x2(acc[hg][dt][0] * f, acc[hg][dt][1] * f),
                                                                pack_f16x2(acc[hg][dt][2] * f, acc[hg][dt][3] * f));
      if (hg == dw && g == 0 && h_base + hl < Hpad)
        *(float4*)(pml + (prow0 + hl) * 4) = make_float4(Ms[hl], Ls[hl], amax, 0.f);
    }
  }
  __syncthreads();
  store_rows((uint16_t*)a.part + prow0 * kD, kD, min(64, Hpad - h_base));
}

// 16-head variant for small query batches: a block owns one query, one head group of 16 and a
// range of tiles, so with one block per (query, head group) no key split (and no combine) is
// needed.  Producers are the same as in the 64-head kernel.  Consumer c computes the partial
// scores of key block c & 1 over dims [256 (c >> 1), +256), the four partials meet in LDS, and
// every consumer runs the same softmax on the summed scores, so P^T and the rescale factors never
// cross waves.  Consumer c then accumulates output dims [128c, 128c+128).  One barrier per tile:
// iteration k runs the softmax and P.V of tile k and the partial scores of tile k+1.
template <int WF, int CF, bool NTG, bool SEL = false>
__global__ __launch_bounds__(kAttnThreads, 1) void attn_bf16_h16_kernel(AttnArgs a, TopkArgs t) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int q = blockIdx.x, split = blockIdx.z;   // grid (query, head block, split)
  const int Hpad = (a.H + 15) & ~15;
  const int h_base = blockIdx.y * 16;
  const int h = h_base + n;   // this lane's head

  __shared__ __align__(16) uint16_t Kr[3][kTile * kKrStride];   // ring of three bf16 row tiles
  __shared__ __align__(16) v4f Sp[2][4][64];                     // partial scores [tile & 1][consumer]
  __shared__ float Xs[4][16];
  __shared__ __align__(16) uint64_t codes[kMaxSlots];
  __shared__ uint32_t vmask[kMaxSlots / kTile];

  const int n_idx = a.n_win + a.n_comp;
  const int n_tiles = (n_idx + kTile - 1) / kTile;
  const int tps = a.tiles_per_split;
  const int t_begin = split * tps;
  const int nt = attn_block_tiles(a, q, n_tiles, t_begin, tps);
  // the fused selection runs only for decode with one query per request (attn_select_fused)
  const int r = SEL ? q : (a.req_mode == 1 ? q / a.q_per_req : (a.req_mode == 2 ? 0 : a.q_req[q]));

  const int kb = wave & 1, dh = wave >> 1;   // consumer roles (waves 0-3)
  // q as the QK B operand: lane (n, g) holds dims 256 dh + 32ks + 8g .. +7 of head h (padded heads
  // read head 0's row; their results are never written)
  // loaded after the slot codes are resolved: the barrier that publishes the codes waits for every
  // outstanding load, and the producers' first gathers should not wait for q
  v8bf qop[8];
  auto load_q = [&] {
    const uint16_t* qp = (const uint16_t*)a.q + ((int64_t)q * a.H + (h < a.H ? h : 0)) * kD + 256 * dh + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qop[ks] = *(const v8bf*)(qp + 32 * ks);
  };
  const int32_t* idx_list = nullptr;
  const int32_t* rows_list = nullptr;
  if constexpr (SEL) {
    // the long rows' selection from the indexer's sketches, into LDS borrowed from ring slots 1-2;
    // q does not depend on it, so its loads overlap it
    if (wave < 4) load_q();
    uint8_t* lds = (uint8_t*)&Kr[0][0];
    select_rows_sketch<kSelSketchPer>(t, q, lds, split == 0 && blockIdx.y == 0, [] {});
    idx_list = (const int32_t*)(lds + kSelListOff);
    rows_list = (const int32_t*)(lds + kSelRowsOff);
  }
  resolve_codes<kAttnThreads>(a, q, r, t_begin * kTile, nt * kTile, codes, vmask, tid, idx_list, rows_list);
  __syncthreads();
  if constexpr (!SEL) {
    if (wave < 4) load_q();
  }

  float m = kNegBig, lsum = 0.f;   // softmax state of head h (identical in the four consumers)
  v4f acc[8];                      // O^T[128 wave + 16 dt + 4 g + i][head h]
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) acc[dt] = v4f{0.f, 0.f, 0.f, 0.f};

  if (wave >= 4) {
    produce_tiles<WF, CF, NTG>(codes, Kr, nt, nt + 2, lane, wave);
  } else {
    const float sc = a.softmax_scale * kLog2e;
    // partial S^T[key 16 kb + 4g + i][head h] over this consumer's 256 dims
    auto qk = [&](const uint16_t* K) {
      v4f x = v4f{0.f, 0.f, 0.f, 0.f};
      const uint16_t* kp = &K[(16 * kb + n) * kKrStride + 256 * dh + 8 * g];
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) x = mma_bf16(*(const v8bf*)(kp + 32 * ks), qop[ks], x);
      return x;
    };
    __syncthreads();                             // barrier 0: tile 0 staged
    if (nt > 0) Sp[0][wave][lane] = qk(Kr[0]);
    __syncthreads();                             // barrier 1: tile 1 staged, scores of tile 0 posted
    int cur = 0;                                 // k % 3
    for (int k = 0; k < nt; ++k) {
      const int pb = k & 1;
      const v4f s0 = Sp[pb][0][lane] + Sp[pb][2][lane];
      const v4f s1 = Sp[pb][1][lane] + Sp[pb][3][lane];
      const uint32_t vm = vmask[k];
      float sv[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sv[i] = (vm >> (4 * g + i)) & 1u ? s0[i] * sc : -INFINITY;
        sv[4 + i] = (vm >> (16 + 4 * g + i)) & 1u ? s1[i] * sc : -INFINITY;
      }
      float tmax = sv[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) tmax = fmaxf(tmax, sv[e]);
      tmax = row_group_max(tmax);
      // lazy rescaling as in the 64-head kernel; alpha is this lane's own head's
      const bool grow = tmax > m + kRescaleLog2;
      if (__builtin_expect(__any(grow), 0)) {
        __asm__ volatile("" ::: "memory");
        const float m_new = grow ? tmax : m;
        const float alpha = exp2f(m - m_new);
        lsum *= alpha;
        m = m_new;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) acc[dt] *= alpha;
      }
      float p[8], psum = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = __builtin_amdgcn_exp2f(sv[e] - m);
        psum += p[e];
      }
      lsum += psum;
      // slot 8g+4mt+i of the K step <-> key 16mt+4g+i: this lane's part of the P^T operand
      const v8bf pf = __builtin_bit_cast(v8bf, make_uint4(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                                                          pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])));
      const uint16_t* K = Kr[cur];
      const uint16_t* tr_lo = &K[(4 * g + (n >> 2)) * kKrStride + 4 * (n & 3) + 128 * wave];
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const v4s lo = lds_read_tr16(tr_lo + 16 * dt);
        const v4s hi = lds_read_tr16(tr_lo + 16 * kKrStride + 16 * dt);
        const v8bf vv = __builtin_bit_cast(v8bf, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        acc[dt] = mma_bf16(vv, pf, acc[dt]);
      }
      cur = cur == 2 ? 0 : cur + 1;
      if (k + 1 < nt) Sp[pb ^ 1][wave][lane] = qk(Kr[cur]);
      __syncthreads();                           // barrier k + 2
    }
  }
  const float ltot = row_group_sum(lsum);
  const int dbase = 128 * wave + 4 * g;
  if (a.n_split == 1) {
    if (wave >= 4 || h >= a.H) return;
    const float sk = a.sink[h] * kLog2e;
    const float M = fmaxf(m, sk);
    const float f = exp2f(m - M);
    const float inv = f / (ltot * f + exp2f(sk - M));
    const int64_t ob = ((int64_t)q * a.H + h) * kD + dbase;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
      store4(a.out, a.out_dt, ob + 16 * dt, acc[dt][0] * inv, acc[dt][1] * inv, acc[dt][2] * inv, acc[dt][3] * inv);
    return;
  }
  // split-K partial: m, l, amax = max |acc| over the head's 512 dims (fp32), acc / amax as fp16
  if (wave < 4) {
    float mx = 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, fabsf(acc[dt][i]));
    mx = row_group_max(mx);
    if (g == 0) Xs[wave][n] = mx;
  }
  __syncthreads();
  if (wave >= 4) return;
  const float amax = fmaxf(fmaxf(Xs[0][n], Xs[1][n]), fmaxf(Xs[2][n], Xs[3][n]));
  const float f = amax > 0.f ? 1.f / amax : 0.f;
  const int64_t prow = ((int64_t)q * a.n_split + split) * Hpad + h;
  uint16_t* pa = (uint16_t*)a.part + prow * kD + dbase;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
    *(uint2*)(pa + 16 * dt) = make_uint2(pack_f16x2(acc[dt][0] * f, acc[dt][1] * f),
                                         pack_f16x2(acc[dt][2] * f, acc[dt][3] * f));
  if (wave == 0 && g == 0) {
    float* pml = (float*)((uint8_t*)a.part + (size_t)a.Q * a.n_split * Hpad * kD * sizeof(uint16_t));
    *(float4*)(pml + prow * 4) = make_float4(m, ltot, amax, 0.f);
  }
}

// Merge split-K partials: out = sum_s 2^(m_s-M) amax_s o_s / (sum_s 2^(m_s-M) l_s + 2^(sink-M)),
// o_s the fp16 partial (acc_s / amax_s).  A thread owns 8 dims of one head and merges groups of
// kCombineGroup splits, every partial of a group loaded up front (the group loop is unrolled and
// predicated); a later group rescales what the earlier ones summed when it raises the max.
constexpr int kCombineGroup = 8;

// merges split groups starting at s_first, every s_step splits, into (M, den, o)
__device__ __forceinline__ void merge_split_groups(const AttnArgs& a, int q, int h, int d, int s_first, int s_step,
                                                   float& M, float& den, float* o) {
  const int Hpad = (a.H + 15) & ~15;
  const uint16_t* p16 = (const uint16_t*)a.part;
  const float* ml = (const float*)((const uint8_t*)a.part + (size_t)a.Q * a.n_split * Hpad * kD * sizeof(uint16_t));
#pragma unroll 1
  for (int s0 = s_first; s0 < a.n_split; s0 += s_step) {
    float4 mls[kCombineGroup];
    uint4 x[kCombineGroup];
#pragma unroll
    for (int i = 0; i < kCombineGroup; ++i) {
      const int sc = s0 + i < a.n_split ? s0 + i : s0;
      const int64_t prow = ((int64_t)q * a.n_split + sc) * Hpad + h;
      mls[i] = *(const float4*)(ml + prow * 4);
      x[i] = *(const uint4*)(p16 + prow * kD + d);
    }
    float Mg = M;
#pragma unroll
    for (int i = 0; i < kCombineGroup; ++i)
      if (s0 + i < a.n_split) Mg = fmaxf(Mg, mls[i].x);
    const float r = exp2f(M - Mg);
    den *= r;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] *= r;
    M = Mg;
#pragma unroll
    for (int i = 0; i < kCombineGroup; ++i) {
      if (s0 + i < a.n_split) {
        const float w = exp2f(mls[i].x - M);
        den = fmaf(w, mls[i].y, den);
        const float wa = w * mls[i].z;
        const uint32_t xs[4] = {x[i].x, x[i].y, x[i].z, x[i].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const v2f v = unpack_f16x2(xs[e]);
          o[2 * e] = fmaf(wa, v[0], o[2 * e]);
          o[2 * e + 1] = fmaf(wa, v[1], o[2 * e + 1]);
        }
      }
    }
  }
}

__device__ __forceinline__ void store_merged(const AttnArgs& a, int q, int h, int d, float den, const float* o) {
  const float inv = 1.f / den;
  const int64_t ob = ((int64_t)q * a.H + h) * kD + d;
  store4(a.out, a.out_dt, ob, o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv);
  store4(a.out, a.out_dt, ob + 4, o[4] * inv, o[5] * inv, o[6] * inv, o[7] * inv);
}

// Block = one query, four heads (a wave per head); used up to kCombineGroup splits.
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
  const int q = blockIdx.x % a.Q, h = (blockIdx.x / a.Q) * 4 + (threadIdx.x >> 6);
  if (h >= a.H) return;
  const int d = (threadIdx.x & 63) * 8;
  float M = a.sink[h] * kLog2e, den = 1.f;   // den holds 2^(sink - M) plus the merged splits' terms
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  merge_split_groups(a, q, h, d, 0, kCombineGroup, M, den, o);
  store_merged(a, q, h, d, den, o);
}

// More splits (long index lists): block = one (query, head); wave w merges split groups w, w + 4,
// ..., so four group chains run side by side, and wave 0 merges the four states through LDS.  Only
// wave 0 starts from the sink term; the others start empty (max -1e30, nothing summed).
__global__ __launch_bounds__(256) void attn_combine_wide_kernel(AttnArgs a) {
  const int q = blockIdx.x % a.Q, h = blockIdx.x / a.Q;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int d = lane * 8;
  __shared__ float sm[4], sden[4];
  __shared__ float so[4][8][64];   // [wave][dim e][lane]: conflict-free writes and reads
  const float sk = a.sink[h] * kLog2e;
  float M = wave == 0 ? sk : kNegBig, den = wave == 0 ? 1.f : 0.f;
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  merge_split_groups(a, q, h, d, wave * kCombineGroup, 4 * kCombineGroup, M, den, o);
  if (lane == 0) {
    sm[wave] = M;
    sden[wave] = den;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) so[wave][e][lane] = o[e];
  __syncthreads();
  if (wave != 0) return;
  const float Mt = fmaxf(fmaxf(sm[0], sm[1]), fmaxf(sm[2], sm[3]));
  float f[4], dt = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    f[w] = exp2f(sm[w] - Mt);
    dt = fmaf(sden[w], f[w], dt);
  }
  float ot[8];
#pragma unroll
  for (int e = 0; e < 8; ++e)
    ot[e] = (so[0][e][lane] * f[0] + so[1][e][lane] * f[1]) + (so[2][e][lane] * f[2] + so[3][e][lane] * f[3]);
  store_merged(a, q, h, d, dt, ot);
}

// fp32 path: block = (query, head); all arithmetic in fp32.
template <bool QBF16>
__global__ __launch_bounds__(256) void attn_f32_kernel(AttnArgs a) {
  const int q = blockIdx.x, h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ float S[4096];
  __shared__ float red[4 * kD];
  __shared__ float s_stat[4];
  const int n_idx = a.n_win + a.n_comp;
  const int r = a.req_mode == 1 ? q / a.q_per_req : (a.req_mode == 2 ? 0 : a.q_req[q]);
  float qv[8];
  if constexpr (QBF16) {
    const uint16_t* qrow = (const uint16_t*)a.q + ((int64_t)q * a.H + h) * kD;
#pragma unroll
    for (int e = 0; e < 8; ++e) qv[e] = bf16_bits_to_f32(qrow[8 * lane + e]);
  } else {
    const float* qrow = (const float*)a.q + ((int64_t)q * a.H + h) * kD;
#pragma unroll
    for (int e = 0; e < 8; ++e) qv[e] = qrow[8 * lane + e];
  }

  float lmax = -INFINITY;
  for (int j = wave; j < n_idx; j += 4) {
    const RowSrc rs = resolve_slot(a, q, r, j);
    float s = -INFINITY;
    if (rs.p != nullptr) {
      float v[8];
      load_chunk8(rs.p, rs.fmt, lane, v);
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) d = fmaf(qv[e], v[e], d);
      s = wave_sum(d) * a.softmax_scale;
    }
    if (lane == 0) S[j] = s;
    lmax = fmaxf(lmax, s);
  }
  if (lane == 0) s_stat[wave] = lmax;
  __syncthreads();
  const float sink = a.sink[h];
  const float M = fmaxf(fmaxf(fmaxf(s_stat[0], s_stat[1]), fmaxf(s_stat[2], s_stat[3])), sink);
  __syncthreads();
  float lsum = 0.f;
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j = wave; j < n_idx; j += 4) {
    const float s = S[j];
    if (s == -INFINITY) continue;
    const float p = expf(s - M);
    lsum += p;
    const RowSrc rs = resolve_slot(a, q, r, j);
    float v[8];
    load_chunk8(rs.p, rs.fmt, lane, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = fmaf(p, v[e], o[e]);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[wave * kD + 8 * lane + e] = o[e];
  if (lane == 0) s_stat[wave] = lsum;
  __syncthreads();
  const float den = s_stat[0] + s_stat[1] + s_stat[2] + s_stat[3] + expf(sink - M);
  for (int d = tid; d < kD; d += 256) {
    const float x = (red[d] + red[kD + d]) + (red[2 * kD + d] + red[3 * kD + d]);
    const float y = x / den;
    if (a.out_dt == 0) ((float*)a.out)[((int64_t)q * a.H + h) * kD + d] = y;
    else ((uint16_t*)a.out)[((int64_t)q * a.H + h) * kD + d] = (uint16_t)f32_to_bf16_bits(y);
  }
}

// The selection runs inside the 64-head attention blocks when its rows fit one block of them
// (at most 16,384 visible entries, the index list at most kMaxSlots slots).
static bool attn_select_fused(const AttnArgs& a, int hb) {
  static const int mode = [] {
    const char* e = getenv("CSA_ATTN_SELECT");   // tuning override: 0 = separate selection launch
    return e ? atoi(e) : -1;
  }();
  const TopkArgs* t = a.sel;
  if (mode == 0 || t == nullptr || t->win_mode != 1 || t->q_per_req != 1 || t->k > kSingleMaxK ||
      a.n_win != kWin || a.n_comp != t->k || a.n_win + a.n_comp > kMaxSlots || t->rows == nullptr)
    return false;
  if (t->sk_top != nullptr)   // long rows: 16-head blocks select from the sketches
    return hb == 16 && topk_sketch_waves(t->max_n_vis) * kSketchTop <= kAttnThreads * kSelSketchPer;
  return hb == 64 && t->max_n_vis <= kSelRowMax;
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  const bool mc = attn_uses_matrix_cores(a.q_dt, a.win_fmt, a.comp_fmt, a.n_win, a.n_comp);
  const int Hpad = (a.H + 15) & ~15;
  const int hb = attn_head_block(a.Q, a.H, a.n_win + a.n_comp);
  const int hchunks = (Hpad + hb - 1) / hb;
  const bool fuse = mc && attn_select_fused(a, hb);
  if (a.sel && !fuse) {
    const hipError_t e = a.sel->sk_top ? launch_topk_sketch(*a.sel, s) : launch_topk_single(*a.sel, s);
    if (e != hipSuccess) return e;
  }
  if (!mc) {
    ProfScope p("attn_f32", s);
    if (a.q_dt == 1) CSA_LAUNCH(p, attn_f32_kernel<true>, dim3((unsigned)a.Q, (unsigned)a.H), dim3(256), s, a);
    else CSA_LAUNCH(p, attn_f32_kernel<false>, dim3((unsigned)a.Q, (unsigned)a.H), dim3(256), s, a);
    return hipGetLastError();
  }
  // a source with no slots takes the other source's format (its loads are never issued)
  const int wf = a.n_win > 0 ? a.win_fmt : a.comp_fmt;
  const int cf = a.n_comp > 0 ? a.comp_fmt : wf;
  {
    ProfScope p(fuse ? "attn_select" : "attn_bf16", s);
    const dim3 grid((unsigned)a.Q, (unsigned)hchunks, (unsigned)a.n_split);
    AttnArgs ak = a;
    const int n_tiles = (a.n_win + a.n_comp + kTile - 1) / kTile;
    ak.tiles_per_split = (n_tiles + a.n_split - 1) / a.n_split;
    const TopkArgs t = fuse ? *a.sel : TopkArgs{};
    // rows are streamed (non-temporal) only when one block gathers each of them: with several head
    // blocks per query, the later blocks' gathers of a row hit the copy the first one left in L2
    const bool stream = a.stream_rows && hchunks == 1;
#define CSA_ATTN_FMT(K, ...)                                                                                       \
  if (wf == kRowFP8 && cf == kRowFP8) CSA_LAUNCH(p, (K<kRowFP8, kRowFP8, __VA_ARGS__>), grid, dim3(kAttnThreads), s, ARGS); \
  else if (wf == kRowFP8) CSA_LAUNCH(p, (K<kRowFP8, kRowBF16, __VA_ARGS__>), grid, dim3(kAttnThreads), s, ARGS);           \
  else if (cf == kRowFP8) CSA_LAUNCH(p, (K<kRowBF16, kRowFP8, __VA_ARGS__>), grid, dim3(kAttnThreads), s, ARGS);           \
  else CSA_LAUNCH(p, (K<kRowBF16, kRowBF16, __VA_ARGS__>), grid, dim3(kAttnThreads), s, ARGS);
    if (hb == 16) {
#define ARGS ak, t
      if (fuse) {
        if (stream) { CSA_ATTN_FMT(attn_bf16_h16_kernel, true, true) } else { CSA_ATTN_FMT(attn_bf16_h16_kernel, false, true) }
      } else {
        if (stream) { CSA_ATTN_FMT(attn_bf16_h16_kernel, true, false) } else { CSA_ATTN_FMT(attn_bf16_h16_kernel, false, false) }
      }
#undef ARGS
    } else {
#define ARGS ak, t
      if (fuse) {
        if (stream) { CSA_ATTN_FMT(attn_bf16_kernel, true, true) } else { CSA_ATTN_FMT(attn_bf16_kernel, false, true) }
      } else {
        if (stream) { CSA_ATTN_FMT(attn_bf16_kernel, true, false) } else { CSA_ATTN_FMT(attn_bf16_kernel, false, false) }
      }
#undef ARGS
    }
#undef CSA_ATTN_FMT
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_split == 1) return e;
  ProfScope p("attn_combine", s);
  if (a.n_split <= kCombineGroup)
    CSA_LAUNCH(p, attn_combine_kernel, dim3((unsigned)(a.Q * ((a.H + 3) / 4))), dim3(256), s, a);
  else
    CSA_LAUNCH(p, attn_combine_wide_kernel, dim3((unsigned)(a.Q * a.H)), dim3(256), s, a);
  return hipGetLastError();
}

CSA_DBG_ACCESSOR(debug_take_violations_attention)

}  // namespace csa
