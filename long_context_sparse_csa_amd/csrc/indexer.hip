// C4 indexer kernels on gfx950: decode (one or several queries per request, keys streamed from
// HBM into registers), causal prefill (keys staged in LDS and shared by a block of queries) and
// the fp32 path.  The page score itself (operand layouts, FP8 through the bf16 matrix cores, FP4
// through the scaled instruction, ReLU and head weights) lives in indexer_score.h.
#include <cstdlib>

#include "indexer_score.h"

namespace csa {

template <bool HIST>
__device__ __forceinline__ void flush_hist(uint32_t* lhist, uint32_t* ghist, int tid) {
  if constexpr (HIST) {
    __syncthreads();
    for (int i = tid; i < kHistBins; i += 256) {
      uint32_t v = lhist[i];
      if (v) atomicAdd(&ghist[i], v);
    }
  }
}


// Pages (64 entries each) scored by one wave, and page buffers in flight per wave.  Measured on the
// batched and long-context decode workloads: 2 pages per wave is 15% slower than 4, 8 matches 4 on
// the first and is 4% faster on the second (and 4 pages per wave for rows without a sketch is no
// faster with the bf16 FP8 path either).  The FP8 path's resident bf16 query operands leave room
// for two page buffers at two waves per SIMD (about 200 VGPRs; three buffers measured 2-7% slower,
// and three waves per SIMD need spills that cost a third more time).
template <bool FP4>
constexpr int kPagesPerWave = FP4 ? 8 : 8;
template <bool FP4>
constexpr int kPageBufs = FP4 ? 3 : 2;
constexpr int kMaxSharedQueries = 4;   // multi-query decode: queries sharing a block's key pages

// NQ > 1 (multi-query decode): the block takes the NQ queries of one request (the last NQ tokens
// of its context).  Wave w scores query w % NQ over page group w / NQ, so every wave does the
// one-query work with the one-query registers, and the NQ waves of a page group read the same
// key pages at the same time: the first read comes from HBM, the others from the caches (the key
// loads keep their lines for NQ > 1).  A block has 4 / NQ page groups (3 waves for NQ = 3).
// Scoring all NQ queries in each wave instead (one key read per page) needs NQ sets of bf16 query
// operands, 256 VGPRs at one wave per SIMD: measured on batched decode with 64 heads, S = 4 took
// 43.8 us that way against 37.2 us this way, S = 2 25.2 against 23.8 us.
template <int NQ>
constexpr int kQGroups = 4 / NQ;

// What the decode kernel leaves for the selection besides the scores: nothing, a per-row 12-bit
// histogram of the scores (the multi-launch selection of rows of any length), or a per-wave sketch
// (the one-launch selection of long rows; see sketch_wave below).
enum SelOut : int { kSelNone = 0, kSelHist = 1, kSelSketch = 2 };

// Per-wave sketch of a long row: the wave's 8 largest scores (order keys and entry indices, in
// ascending index order) and the 9th largest order key, an upper bound for every entry of the wave
// left out.  The selection takes the k largest of all waves' sketches; a wave whose bound reaches
// the k-th of them may hide a selected entry, and only then are the full scores read back.
//   Each lane holds one entry of each of the wave's 8 pages.  It sorts its 8 (key, page) pairs
// (descending keys, a 19-exchange network), then 8 rounds take the wave's largest lane head (the
// lowest lane on ties: within a wave the order of equal keys is immaterial, because a left-out entry
// equal to a kept one makes the bound reach it) and that lane advances; a 9th round reads the
// bound.  Entries past the visible prefix carry key 0 and page code 15 and give index -1.

__device__ __forceinline__ void sketch_wave(const uint32_t* key8, uint32_t valid8, int64_t e_base, int lane,
                                            uint2* top, uint32_t* bound) {
  uint32_t k[8], pg[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const bool v = (valid8 >> i) & 1u;
    k[i] = v ? key8[i] : 0u;
    pg[i] = v ? (uint32_t)i : 15u;
  }
  auto cx = [&](int x, int y) {   // descending: larger key to x
    const bool sw = k[y] > k[x];
    const uint32_t kx = k[x], ky = k[y], px = pg[x], py = pg[y];
    k[x] = sw ? ky : kx; k[y] = sw ? kx : ky;
    pg[x] = sw ? py : px; pg[y] = sw ? px : py;
  };
  // Batcher's odd-even merge sort of 8
  cx(0, 1); cx(2, 3); cx(4, 5); cx(6, 7);
  cx(0, 2); cx(1, 3); cx(4, 6); cx(5, 7);
  cx(1, 2); cx(5, 6);
  cx(0, 4); cx(1, 5); cx(2, 6); cx(3, 7);
  cx(2, 4); cx(3, 5);
  cx(1, 2); cx(3, 4); cx(5, 6);
  uint32_t my_key = 0u, my_idx = 0xFFFFFFFFu;
#pragma unroll
  for (int r = 0; r < kSketchTop; ++r) {
    const uint32_t kmax = wave_umax(k[0]);
    const int win = __builtin_ctzll(__ballot(k[0] == kmax));
    const uint32_t cand = pg[0] < 8u ? (uint32_t)(e_base + (int64_t)pg[0] * kPage) : 0xFFFFFFFFu;
    const uint32_t idx_r = (uint32_t)__builtin_amdgcn_readlane((int)cand, win);
    my_key = lane == r ? kmax : my_key;
    my_idx = lane == r ? idx_r : my_idx;
    const bool adv = lane == win;
#pragma unroll
    for (int i = 0; i < 7; ++i) {
      k[i] = adv ? k[i + 1] : k[i];
      pg[i] = adv ? pg[i + 1] : pg[i];
    }
    k[7] = adv ? 0u : k[7];
    pg[7] = adv ? 15u : pg[7];
  }
  const uint32_t bnd = wave_umax(k[0]);
  // lanes 0-7 hold the kept entries; each lands at its rank by index (index -1, as unsigned, last)
  int rank = 0;
#pragma unroll
  for (int s2 = 0; s2 < kSketchTop; ++s2) {
    const uint32_t o = (uint32_t)__builtin_amdgcn_readlane((int)my_idx, s2);
    rank += (o < my_idx || (o == my_idx && s2 < lane)) ? 1 : 0;
  }
  if (lane < kSketchTop) top[rank] = make_uint2(my_key, my_idx);
  if (lane == 0) *bound = bnd;
}

// FP8 operands run at two waves per SIMD (the resident query operands and two page buffers take
// about 190 VGPRs); stating that occupancy to the compiler (amdgpu_waves_per_eu) changes its
// schedule and measured faster: long-context indexer 50.0 -> 48.2 us, batched 17.0 -> 16.5 us
// (interleaved, one box).  FP4 fits three waves (about 150 VGPRs), and capping it at two cost its
// long-context launch 1.4 us, so its bound stays three.
template <int NHG, int SEL, bool FP4, int NQ>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, FP4 ? 3 : 2))) void indexer_fp8_kernel(
    IndexerArgs a) {
  constexpr bool HIST = SEL == kSelHist;
  constexpr bool SK = SEL == kSelSketch;
  constexpr int pages_per_wave = kPagesPerWave<FP4>;
  static_assert(!SK || pages_per_wave * kPage == kSketchSpan, "a sketch covers one wave's pages");
  constexpr int nbuf = kPageBufs<FP4> < pages_per_wave ? kPageBufs<FP4> : pages_per_wave;
  constexpr int kGroups = kQGroups<NQ>;
  const int q0 = blockIdx.x * NQ;   // queries vary fastest: a row's blocks share one XCD (and its L2)
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int jq = wave % NQ, grp = wave / NQ;   // this wave's query and page group
  const int n = lane & 15, g = lane >> 4;
  __shared__ uint32_t lhist[HIST ? NQ : 1][HIST ? kHistBins : 1];

  const int64_t c_begin = (int64_t)blockIdx.y * kGroups * pages_per_wave * kPage;
  if (c_begin >= a.max_n_vis) return;
  int r;
  int64_t nv = 0, nv_max = 0;   // visible entries of this wave's query, and the block's largest
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    const int64_t v = visible_count(a, q0 + j, r);   // one request: every j gives the same r
    nv_max = v > nv_max ? v : nv_max;
    nv = j == jq ? v : nv;
  }
  // inside a fused path the selection reads only the visible prefix of each row, so a block (or
  // a wave, below) past it has nothing to do; short rows of a ragged batch then cost nothing
  if (a.visible_only && c_begin >= nv_max) return;
  if constexpr (HIST) {
    // the waves of a query add into its part of the histogram, so all clears must land before
    // the first add (both returns above are block-uniform, so every wave reaches this barrier)
    for (int i = tid; i < NQ * kHistBins; i += (int)blockDim.x) lhist[i / kHistBins][i % kHistBins] = 0u;
    __syncthreads();
  }

  // A operands: the query's indexer heads, resident in VGPRs.  Loads are unconditional (clamped
  // addresses, padded heads zeroed by select) so nothing waits before the first key page.
  const int q = q0 + jq;
  QueryOps<NHG, FP4> qo;
  load_query<NHG, FP4>(a, q, n, g, qo);

  const uint8_t* keys = (const uint8_t*)a.keys;
  const int32_t* pt = a.page_table + (int64_t)(r < 0 ? 0 : r) * a.max_pages;
  const int64_t p_first = (c_begin >> 6) + (int64_t)grp * pages_per_wave;   // this wave's first page
  const int64_t vis_pages = (nv + kPage - 1) / kPage;

  // page ids of this wave's pages, one per lane, then read into scalars as needed
  int my_pid = -1;
  {
    const int64_t pp = p_first + lane;
    if (lane < pages_per_wave && pp < vis_pages) my_pid = pt[pp];
  }

  // key page p -> operands; invalid pages read page 0 (always mapped memory) and are masked later
  auto page_ok = [&](int i) {
    const int pid = __builtin_amdgcn_readlane(my_pid, i);
    return (unsigned)pid < (unsigned)a.num_pages;
  };
  auto load_page = [&](int i, v8i* kb, uint32_t& ks_lo, uint32_t& ks_hi) {
    int pid = __builtin_amdgcn_readlane(my_pid, i);
    pid = (unsigned)pid < (unsigned)a.num_pages ? pid : 0;
    const uint8_t* kp = keys + (int64_t)pid * (kPage * kRowB<FP4>) + 16 * lane;
    page_scale_words<FP4>(a.kscale + (int64_t)pid * 256, n, g, ks_lo, ks_hi);
#pragma unroll
    for (int kg = 0; kg < 4; ++kg) kb[kg] = load_key_operand<FP4, NQ == 1>(kp, kg);
  };

  // a long sketch row stores no scores (wave-uniform); its selection rescores it if it must
  const bool no_store = SK && a.sk_rescore_from > 0 && nv >= a.sk_rescore_from;
  uint32_t skey[SK ? pages_per_wave : 1];   // sketch: order key of this lane's entry of page i
  uint32_t svalid = 0u;                      // bit i: that entry is visible
  auto compute_page = [&](int i, const v8i* kb, uint32_t ks_lo, uint32_t ks_hi) {
    const int64_t c0 = (p_first + i) * kPage;
    const bool mapped = page_ok(i);
    const int64_t c = c0 + 4 * n + g;
    CSA_DBG_COUNT(lane == 0 && !mapped && c0 < nv);   // a visible page with no page id in the pool
    const float score = score_page<NHG, FP4>(qo, kb, ks_lo, ks_hi);
    const float v = (mapped && c0 < nv && c < nv) ? score : -INFINITY;
    if (c < (a.visible_only ? nv : a.max_n_vis) && !no_store) {
      a.logits[(int64_t)q * a.ld + c] = v;
      if constexpr (HIST) {
        if (c < nv) atomicAdd(&lhist[jq][order_key(v) >> kHistShift], 1u);
      }
    }
    if constexpr (SK) {
      skey[i] = order_key(v);
      svalid |= (c < nv ? 1u : 0u) << i;
    }
  };

  // nbuf page buffers, straight-line code: the first nbuf pages are loaded up front and page
  // i + nbuf as soon as page i is scored, so up to nbuf pages are in flight and every wait is for
  // exactly the page about to be scored.  Pages past the wave's range load page 0 (always mapped)
  // and store nothing.
  if (!(a.visible_only && p_first * kPage >= nv)) {
    v8i kb[nbuf][4];
    uint32_t ks_lo[nbuf], ks_hi[nbuf];
#pragma unroll
    for (int i = 0; i < nbuf; ++i) load_page(i, kb[i], ks_lo[i], ks_hi[i]);
#pragma unroll
    for (int i = 0; i < pages_per_wave; ++i) {
      compute_page(i, kb[i % nbuf], ks_lo[i % nbuf], ks_hi[i % nbuf]);
      if (i + nbuf < pages_per_wave) load_page(i + nbuf, kb[i % nbuf], ks_lo[i % nbuf], ks_hi[i % nbuf]);
    }
    if constexpr (SK) {
      // wave W of the row covers entries [W * kSketchSpan, (W + 1) * kSketchSpan)
      const int64_t W = p_first / pages_per_wave;
      const int64_t slot = (int64_t)q * a.sk_waves + W;
      sketch_wave(skey, svalid, p_first * kPage + 4 * n + g, lane, a.sk_top + slot * kSketchTop, a.sk_bound + slot);
    }
  }
  if constexpr (HIST) {
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      uint32_t* gh = a.hist + (int64_t)(q0 + j) * kHistBins;
      for (int i = tid; i < kHistBins; i += (int)blockDim.x) {
        const uint32_t v = lhist[j][i];
        if (v) atomicAdd(&gh[i], v);
      }
    }
  }
}

// Causal prefill: every query scores the keys of request 0, so keys are shared across queries.  A
// block stages a few key pages in LDS once and scores kPfQueries consecutive queries against them
// (four per wave), instead of every query streaming every page.  Query blocks are issued heaviest
// (latest) first, and only the visible prefix of each row is written: the selection reads nothing
// past it.
//   FP4 keys (indexer_fp4_prefill_kernel): kPfPages pages (24 KB) and their scale words are staged
// in operand order, [page][key group kg][lane][16 B], with direct global-to-LDS loads (each lane
// fetches the chunk that belongs at its 16-byte slot, so no registers hold keys in transit), and
// every LDS read of an operand is 64 lanes x 16 contiguous bytes.  The kernel is bound by the
// matrix-core / VALU pair of each page score (16 scaled MFMAs and 128 ReLU/weight operations);
// one wave alone leaves both units half idle, so the block is sized for three waves per SIMD
// (measured with FP8 keys on the 8192-token causal prefill before FP8 moved to bf16: 8 pages at
// two waves per SIMD, with next-query prefetch and double-buffered key operands, was 18% slower).
//   FP8 keys (indexer_fp8_prefill_kernel): each wave converts one page to its bf16 operands while
// staging it, [page][key group][MFMA j][lane][16 B] (16 KB a page), so the per-query work is the
// 64 MFMAs and the epilogue, with no conversion.
constexpr int kPfPages = 6;
constexpr int kPfQueries = 16;

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef const __attribute__((address_space(1))) void* gbl_ptr_t;

// entries visible to causal-prefill query q: those with index < floor((pos0 + q + 1) / 4)
__device__ __forceinline__ int64_t prefill_visible(const IndexerArgs& a, int q) {
  const int64_t lim = min<int64_t>(a.max_n_vis, (int64_t)a.max_pages * kPage);
  const int64_t nv = (a.pos0 + q + 1) / 4;
  return a.n_req < 1 ? 0 : (nv > lim ? lim : nv);
}


template <int NHG, bool FP4>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3))) void indexer_fp4_prefill_kernel(
    IndexerArgs a) {
  constexpr int kHalves = FP4 ? 1 : 2;                            // 16-byte chunks per lane operand
  constexpr int kRow = kRowB<FP4>;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int nbx = (a.Q + kPfQueries - 1) / kPfQueries;
  const int q0 = (nbx - 1 - (int)blockIdx.x) * kPfQueries;       // heaviest query blocks first
  const int64_t p0 = (int64_t)blockIdx.y * kPfPages;
  if (p0 * kPage >= a.max_n_vis) return;
  __shared__ __align__(16) uint8_t kl[kPfPages][4][kHalves][64][16];   // [page][kg][half][lane] operand bytes
  __shared__ __align__(16) uint32_t sl[kPfPages][64];             // scale word of lane l = word l
  __shared__ int pid_s[kPfPages];

  const int qw = q0 + 4 * wave;                                   // this wave's first query
  const int nq = min(4, a.Q - qw);                                // its query count (may be <= 0)
  const int qlast = min(q0 + kPfQueries, a.Q) - 1;
  const int64_t nv_last = prefill_visible(a, qlast);              // the largest prefix of the block
  if (p0 * kPage >= nv_last) return;   // no query of the block sees these pages

  if (tid < kPfPages) {
    const int64_t pp = p0 + tid;
    int pid = -1;
    if (pp * kPage < nv_last) pid = a.page_table[pp];
    pid_s[tid] = pid;
  }
  __syncthreads();
  // wave w stages pages w and w + 4: 4 x kHalves contiguous 1 KB loads per page (the page is in
  // operand order, so load j is key group j / kHalves, half j % kHalves), then its 256 scale bytes
  const uint8_t* keys = (const uint8_t*)a.keys;
  for (int pg = wave; pg < kPfPages; pg += 4) {
    int pid = pid_s[pg];
    pid = (unsigned)pid < (unsigned)a.num_pages ? pid : 0;
    const uint8_t* kp = keys + (int64_t)pid * (kPage * kRow) + 16 * lane;
#pragma unroll
    for (int j = 0; j < 4 * kHalves; ++j) {
      const int kg = j / kHalves, half = j % kHalves;
      __builtin_amdgcn_global_load_lds((gbl_ptr_t)(kp + 1024 * j), (lds_ptr_t)&kl[pg][kg][half][0][0], 16, 0, 0);
    }
    __builtin_amdgcn_global_load_lds((gbl_ptr_t)(a.kscale + (int64_t)pid * 256 + 4 * lane),
                                     (lds_ptr_t)&sl[pg][0], 4, 0, 0);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // bit i: staged page i is mapped (wave-uniform)
  uint32_t live_bits = 0;
#pragma unroll
  for (int i = 0; i < kPfPages; ++i) live_bits |= ((unsigned)pid_s[i] < (unsigned)a.num_pages ? 1u : 0u) << i;
  live_bits = __builtin_amdgcn_readfirstlane(live_bits);

  for (int j = 0; j < nq; ++j) {
    const int q = qw + j;
    const int64_t nv = prefill_visible(a, q);
    float* lrow = a.logits + (int64_t)q * a.ld;
    // pages of this block holding visible entries of q (wave-uniform)
    const int64_t vis_end = nv - p0 * kPage;
    const int np = vis_end <= 0 ? 0 : (int)min<int64_t>((vis_end + kPage - 1) / kPage, kPfPages);
    if (np == 0) continue;
    QueryOps<NHG, FP4> qo;
    load_query<NHG, FP4>(a, q, n, g, qo);
    for (int pi = 0; pi < np; ++pi) {
      v8i kb[4];
      uint32_t ks_lo, ks_hi;
      page_scale_words<FP4>((const uint8_t*)&sl[pi][0], n, g, ks_lo, ks_hi);
#pragma unroll
      for (int kg = 0; kg < 4; ++kg) {
        const uint4 lo = *(const uint4*)&kl[pi][kg][0][lane][0];
        kb[kg][0] = (int)lo.x; kb[kg][1] = (int)lo.y; kb[kg][2] = (int)lo.z; kb[kg][3] = (int)lo.w;
        if constexpr (FP4) {
          kb[kg][4] = 0; kb[kg][5] = 0; kb[kg][6] = 0; kb[kg][7] = 0;
        } else {
          const uint4 hi = *(const uint4*)&kl[pi][kg][kHalves - 1][lane][0];
          kb[kg][4] = (int)hi.x; kb[kg][5] = (int)hi.y; kb[kg][6] = (int)hi.z; kb[kg][7] = (int)hi.w;
        }
      }
      const bool live = (live_bits >> pi) & 1u;
      const float score = score_page<NHG, FP4>(qo, kb, ks_lo, ks_hi);
      const int64_t c = (p0 + pi) * kPage + 4 * n + g;
      if (c < a.max_n_vis) lrow[c] = (live && c < nv) ? score : -INFINITY;
    }
  }
}

// FP8 prefill, query-major: a block of four waves takes four consecutive queries, one per wave,
// and walks the pages they see in chunks of kPqChunk pages.  The four waves convert the next chunk
// to bf16 operands into an LDS double buffer (its loads issued before the current chunk is
// scored, the conversion after) while each wave scores the current chunk for its query, so a
// query's operands are loaded and converted once per block.  Measured on the 8,192-token causal
// prefill: 108 us at one page per chunk and three waves per SIMD (32 KB of LDS a block), 114 us
// at two pages and two waves per SIMD, 130 us for the page-major shape this replaces (a block
// staging four pages for sixteen queries, each query's operands loaded once per page block).
constexpr int kPqChunk = 1;

template <int NHG>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3))) void indexer_fp8_prefill_kernel(
    IndexerArgs a) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int nb = (a.Q + 3) / 4;
  const int q0 = (nb - 1 - (int)blockIdx.x) * 4;   // heaviest (latest) query blocks first
  const int q = q0 + wave;
  const bool has_q = q < a.Q;
  const int64_t nv_last = prefill_visible(a, min(q0 + 3, a.Q - 1));   // the block's largest prefix
  const int64_t n_pages = (nv_last + kPage - 1) / kPage;
  if (n_pages == 0) return;   // block-uniform: no query of the block sees an entry
  const int n_chunks = (int)((n_pages + kPqChunk - 1) / kPqChunk);
  __shared__ v4u kbf[2][kPqChunk][4][4][64];   // [buffer][page][kg][j][lane] bf16 operands
  __shared__ int pid_s[2][kPqChunk];

  // the query's operands first: their loads overlap the first chunk's
  QueryOps<NHG, false> qo;
  if (has_q) load_query<NHG, false>(a, q, n, g, qo);
  const int64_t nv = has_q ? prefill_visible(a, q) : 0;
  float* lrow = a.logits + (int64_t)(has_q ? q : 0) * a.ld;

  // staging: chunk c's (page, key group) pairs t = wave, wave + 4 (kPqChunk * 4 = 8 pairs)
  constexpr int kPairs = kPqChunk * 4 / 4;
  v8i sraw[kPairs];
  uint32_t slo[kPairs], shi[kPairs];
  auto stage_issue = [&](int c, int buf) {
#pragma unroll
    for (int u = 0; u < kPairs; ++u) {
      const int t = wave + 4 * u, i = t >> 2, kg = t & 3;
      const int64_t pp = (int64_t)c * kPqChunk + i;
      int pid = pp < n_pages ? a.page_table[pp] : -1;
      if (kg == 0 && lane == 0) pid_s[buf][i] = pid;
      pid = (unsigned)pid < (unsigned)a.num_pages ? pid : 0;
      const uint8_t* kp = (const uint8_t*)a.keys + (int64_t)pid * (kPage * kDI) + 16 * lane;
      sraw[u] = load_key_operand<false, false>(kp, kg);
      page_scale_words<false>(a.kscale + (int64_t)pid * 256, n, g, slo[u], shi[u]);
    }
  };
  auto stage_finish = [&](int buf) {
#pragma unroll
    for (int u = 0; u < kPairs; ++u) {
      const int t = wave + 4 * u, i = t >> 2, kg = t & 3;
      v8bf o[4];
      fp8_operand_bf16(sraw[u], e8m0_float((slo[u] >> (8 * kg)) & 0xFFu), e8m0_float((shi[u] >> (8 * kg)) & 0xFFu), o);
#pragma unroll
      for (int j = 0; j < 4; ++j) kbf[buf][i][kg][j][lane] = __builtin_bit_cast(v4u, o[j]);
    }
  };
  stage_issue(0, 0);
  stage_finish(0);
  __syncthreads();
  auto qop = [&](int hg, int jj) -> const v8bf& { return qo.bf[hg][jj]; };
  for (int c = 0; c < n_chunks; ++c) {
    const int buf = c & 1;
    // the other buffer was last read in chunk c - 1, before the barrier that ended it
    if (c + 1 < n_chunks) stage_issue(c + 1, buf ^ 1);
#pragma unroll
    for (int i = 0; i < kPqChunk; ++i) {
      const int64_t p = (int64_t)c * kPqChunk + i;
      if (p * kPage < nv) {   // wave-uniform: pages holding visible entries of this query
        float part[4];
#pragma unroll
        for (int kg = 0; kg < 4; ++kg) {
          v8bf kf[4];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) kf[jj] = __builtin_bit_cast(v8bf, kbf[buf][i][kg][jj][lane]);
          part[kg] = key_group_bf16<NHG>(qop, qo.wv, kf);
        }
        const float score = reduce_key_groups(part);
        const bool live = (unsigned)pid_s[buf][i] < (unsigned)a.num_pages;
        const int64_t e = p * kPage + 4 * n + g;
        if (e < a.max_n_vis) lrow[e] = (live && e < nv) ? score : -INFINITY;
      }
    }
    if (c + 1 < n_chunks) stage_finish(buf ^ 1);
    __syncthreads();
  }
}

// fp32 indexer (unquantised queries and keys): 4 threads per entry, heads split between them.
template <bool HIST>
__global__ __launch_bounds__(256) void indexer_f32_kernel(IndexerArgs a) {
  const int q = blockIdx.x;   // queries vary fastest: a row's blocks share one XCD (and its L2)
  const int tid = threadIdx.x;
  __shared__ float qs[64 * kDI];
  __shared__ float ks[kPage * (kDI + 1)];
  __shared__ float ws[64];
  __shared__ uint32_t lhist[HIST ? kHistBins : 1];

  const int64_t c0 = (int64_t)blockIdx.y * kPage;
  if (c0 >= a.max_n_vis) return;
  int r;
  const int64_t nv = visible_count(a, q, r);
  if constexpr (HIST) {
    for (int i = tid; i < kHistBins; i += 256) lhist[i] = 0u;
  }
  const float* qf = (const float*)a.qI + (int64_t)q * a.HI * kDI;
  for (int i = tid; i < a.HI * kDI; i += 256) qs[i] = qf[i];
  if (tid < a.HI) ws[tid] = a.w[(int64_t)q * a.HI + tid];
  int page = -1;
  if (c0 < nv) page = a.page_table[(int64_t)r * a.max_pages + (c0 >> 6)];
  const bool page_ok = (unsigned)page < (unsigned)a.num_pages;
  if (page_ok) {
    const float* kp = (const float*)a.keys + (int64_t)page * kPage * kDI;
    for (int i = tid; i < kPage * kDI; i += 256) ks[(i / kDI) * (kDI + 1) + (i % kDI)] = kp[i];
  }
  __syncthreads();
  const int key = tid >> 2, part = tid & 3;
  float s = 0.f;
  if (page_ok) {
    for (int h = part; h < a.HI; h += 4) {
      float dot = 0.f;
      for (int d = 0; d < kDI; ++d) dot = fmaf(qs[h * kDI + d], ks[key * (kDI + 1) + d], dot);
      s = fmaf(ws[h], fmaxf(dot, 0.f), s);
    }
  }
  s += __shfl_xor(s, 1);
  s += __shfl_xor(s, 2);
  const int64_t c = c0 + key;
  if (part == 0 && c < a.max_n_vis) {
    const float v = (c < nv && page_ok) ? s : -INFINITY;
    a.logits[(int64_t)q * a.ld + c] = v;
    if constexpr (HIST) {
      if (c < nv) atomicAdd(&lhist[order_key(v) >> kHistShift], 1u);
    }
  }
  flush_hist<HIST>(lhist, a.hist + (int64_t)q * kHistBins, tid);
}

hipError_t launch_indexer(const IndexerArgs& a, hipStream_t s) {
  if (a.max_n_vis <= 0) return hipSuccess;
  const bool hist = a.hist != nullptr;
  const bool sketch = a.sk_top != nullptr;
  if (a.dt == 0) {
    dim3 grid((unsigned)a.Q, (unsigned)((a.max_n_vis + kPage - 1) / kPage));
    ProfScope p("indexer_f32", s);
    if (hist) CSA_LAUNCH(p, indexer_f32_kernel<true>, grid, dim3(256), s, a);
    else CSA_LAUNCH(p, indexer_f32_kernel<false>, grid, dim3(256), s, a);
    return hipGetLastError();
  }
  const int nhg = (a.HI + 15) / 16;
  const bool fp4 = a.dt == 3;
  if (a.vis_mode == 2 && !hist) {
    // causal prefill: keys shared by all queries, staged once per block of queries
    // FP4: page-major blocks (kPfPages pages, kPfQueries queries); FP8: query-major blocks of 4
    const dim3 block(256);
    dim3 grid = fp4 ? dim3((unsigned)((a.Q + kPfQueries - 1) / kPfQueries),
                           (unsigned)((a.max_n_vis + kPfPages * kPage - 1) / (kPfPages * kPage)))
                    : dim3((unsigned)((a.Q + 3) / 4));
    ProfScope p(fp4 ? "indexer_fp4_prefill" : "indexer_fp8_prefill", s);
#define CSA_PF_LAUNCH(N)                                                                    \
  if (fp4) CSA_LAUNCH(p, (indexer_fp4_prefill_kernel<N, true>), grid, block, s, a); \
  else CSA_LAUNCH(p, (indexer_fp8_prefill_kernel<N>), grid, block, s, a);
    switch (nhg) {
      case 1: CSA_PF_LAUNCH(1) break;
      case 2: CSA_PF_LAUNCH(2) break;
      case 3: CSA_PF_LAUNCH(3) break;
      default: CSA_PF_LAUNCH(4) break;
    }
#undef CSA_PF_LAUNCH
    return hipGetLastError();
  }
  // kPagesPerWave pages per wave, four waves per block; a multi-query decode (2 to 4 queries per
  // request, derived visibility) gives each block all queries of one request
  const int nq = (a.vis_mode == 1 && a.q_per_req >= 2 && a.q_per_req <= kMaxSharedQueries) ? a.q_per_req : 1;
  const int groups = 4 / nq;   // kQGroups<nq>: page groups per block, nq waves each
  const int per_block = groups * (fp4 ? kPagesPerWave<true> : kPagesPerWave<false>) * kPage;
  dim3 grid((unsigned)(a.Q / nq), (unsigned)((a.max_n_vis + per_block - 1) / per_block));
  const dim3 block((unsigned)(64 * nq * groups));
  ProfScope p(fp4 ? "indexer_fp4" : "indexer_fp8", s);
#define CSA_IDX_LAUNCH(N, F, NQ)                                                                           \
  if (hist) CSA_LAUNCH(p, (indexer_fp8_kernel<N, kSelHist, F, NQ>), grid, block, s, a);             \
  else if (sketch) CSA_LAUNCH(p, (indexer_fp8_kernel<N, kSelSketch, F, NQ>), grid, block, s, a);  \
  else CSA_LAUNCH(p, (indexer_fp8_kernel<N, kSelNone, F, NQ>), grid, block, s, a);
#define CSA_IDX_NQ(N, F)                          \
  switch (nq) {                                   \
    case 2: CSA_IDX_LAUNCH(N, F, 2) break;        \
    case 3: CSA_IDX_LAUNCH(N, F, 3) break;        \
    case 4: CSA_IDX_LAUNCH(N, F, 4) break;        \
    default: CSA_IDX_LAUNCH(N, F, 1) break;       \
  }
#define CSA_IDX_FMT(N) \
  if (fp4) { CSA_IDX_NQ(N, true) } else { CSA_IDX_NQ(N, false) }
  switch (nhg) {
    case 1: CSA_IDX_FMT(1) break;
    case 2: CSA_IDX_FMT(2) break;
    case 3: CSA_IDX_FMT(3) break;
    default: CSA_IDX_FMT(4) break;
  }
#undef CSA_IDX_FMT
#undef CSA_IDX_NQ
#undef CSA_IDX_LAUNCH
  return hipGetLastError();
}

CSA_DBG_ACCESSOR(debug_take_violations_indexer)

}  // namespace csa
