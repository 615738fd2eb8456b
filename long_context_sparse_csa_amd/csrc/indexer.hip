// C4 indexer scores on gfx950.
//
// Score of compressed entry c for one query ([P1] "DeepSeek-V4 全面解读" section 2.10, forward steps
// 5-8; [P2] "DeepSeek-V4 in SGLang 深度理解分析" concept 3 / algorithm 2):
//     s[c] = sum_h w[h] * max(0, qI[h] . kI[c])
// with FP8 E4M3FN or FP4 E2M1 operands that carry one E8M0 scale per 32 elements.
//
// FP8 path: one v_mfma_scale_f32_16x16x128_f8f6f4 covers 16 heads x 16 entries x all 128 dims, and
// its per-lane E8M0 scale operands are exactly the stored per-32 block scales, so dequantisation
// costs nothing.  Operand layout (measured on gfx950): lane l = m + 16*g holds row m, bytes 0..15
// -> k in [16g, 16g+16), bytes 16..31 -> k in [64+16g, 64+16g+16); its scale byte scales row m's
// 32-element block g.  A wave scores one page (64 entries) per step: MFMA column n of key group kg
// is slot 4n+kg, so lane l's scale dword is word l of the page's [4 blocks][64 slots] scale array
// and the key group picks the byte (opsel).  The epilogue applies ReLU and the head weights, then a
// 2-step reduce-scatter over the four lane groups leaves lane l with the full score of slot
// 4*(l%16) + l/16.  Decode: keys stream straight from HBM into VGPRs (no LDS), each lane loads
// 2 x 16 B per key group, and each page is read exactly once.  Causal prefill, where all queries
// share one request's keys, stages key pages in LDS per block of queries instead (see below).
//
// FP4 path (two E2M1 codes per byte, element 2i in the low nibble): the same instruction with both
// operand formats set to FP4 reads four registers per lane, and lane l = m + 16*g's 32 codes all
// fall in scale block g (measured on gfx950).  Lane (m, g) therefore loads the one contiguous
// 16-byte chunk of row m that holds elements [32g, 32g+32), and the scale operands are exactly the
// FP8 path's.  A and B use the same lane layout, so codes pair up element by element.  Rows are
// 64 bytes, a key page 4 KB: half the FP8 key traffic, at the same matrix-core cost per page.
#include <cstdlib>

#include "csa_device.h"
#include "csa_internal.h"

namespace csa {

// bytes of one 128-dim operand row
template <bool FP4>
constexpr int kRowB = FP4 ? kDI / 2 : kDI;

template <int HG, int KG, bool FP4>
__device__ __forceinline__ v4f mma_scaled(const v8i& a, const v8i& b, int sa, int sb, v4f c) {
  constexpr int fmt = FP4 ? 4 : 0;   // operand format code: 0 = fp8 e4m3, 4 = fp4 e2m1
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, fmt, fmt, HG, sa, KG, sb);
}

// max(x, 0) as one integer max on the bit pattern: every negative float (and -0) is a negative
// integer, every other float keeps its bits.  A float max costs two instructions here, because the
// compiler first quiets possible signalling NaNs of the matrix-core result.
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// 16 bytes, optionally as a non-temporal load: decode keys are read exactly once, so streaming
// them without keeping them in L2 leaves the L2 to the score rows the selection reads next
template <bool NT>
__device__ __forceinline__ v4u load16(const uint8_t* p) {
  if constexpr (NT) return __builtin_nontemporal_load((const v4u*)p);
  else return *(const v4u*)p;
}

// One row-major 128-dim row (a query head) as a scaled-MFMA operand: lane (n, g) takes bytes
// [16g, 16g+16) and, for FP8, [64+16g, 64+16g+16) of its row (the same split as the keys below)
template <bool FP4>
__device__ __forceinline__ v8i load_row_operand(const uint8_t* row, int g) {
  const v4u lo = load16<false>(row + 16 * g);
  v8i r;
  r[0] = (int)lo[0]; r[1] = (int)lo[1]; r[2] = (int)lo[2]; r[3] = (int)lo[3];
  if constexpr (FP4) {
    r[4] = 0; r[5] = 0; r[6] = 0; r[7] = 0;
  } else {
    const v4u hi = load16<false>(row + 64 + 16 * g);
    r[4] = (int)hi[0]; r[5] = (int)hi[1]; r[6] = (int)hi[2]; r[7] = (int)hi[3];
  }
  return r;
}

// Index-key pages are stored in operand order: the 16 bytes that lane L = n + 16g takes for key
// group kg and half h (row 4n + kg, bytes [64h + 16g, +16)) sit at byte (kg·halves + h)·1024 + 16L
// of the page, so every load instruction of a page reads one contiguous kilobyte (a row-major
// page would touch sixteen 128-byte lines per quarter-wave instead of two).  `lane_base` is the
// page address plus 16·lane; loads are non-temporal.
template <bool FP4>
__device__ __forceinline__ v8i load_key_operand(const uint8_t* lane_base, int kg) {
  constexpr int halves = FP4 ? 1 : 2;
  const v4u lo = load16<true>(lane_base + kg * halves * 1024);
  v8i r;
  r[0] = (int)lo[0]; r[1] = (int)lo[1]; r[2] = (int)lo[2]; r[3] = (int)lo[3];
  if constexpr (FP4) {
    r[4] = 0; r[5] = 0; r[6] = 0; r[7] = 0;
  } else {
    const v4u hi = load16<true>(lane_base + (kg * halves + 1) * 1024);
    r[4] = (int)hi[0]; r[5] = (int)hi[1]; r[6] = (int)hi[2]; r[7] = (int)hi[3];
  }
  return r;
}

__device__ __forceinline__ int64_t visible_count(const IndexerArgs& a, int q, int& r) {
  int64_t nv;
  if (a.vis_mode == 1) {
    nv = decode_seen(a.ctx_len, a.max_ctx, a.q_per_req, q, r) / 4;
  } else if (a.vis_mode == 2) {
    r = 0;
    nv = (a.pos0 + q + 1) / 4;
  } else {
    r = a.q_req[q];
    nv = a.n_vis[q];
  }
  int64_t lim = a.max_n_vis < (int64_t)a.max_pages * kPage ? a.max_n_vis : (int64_t)a.max_pages * kPage;
  nv = nv < 0 ? 0 : (nv > lim ? lim : nv);
  if (r < 0 || r >= a.n_req) nv = 0;
  return nv;
}

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

// The query's indexer heads as scaled-MFMA A operands (padded heads zeroed), their E8M0 block
// scales packed one byte per head group, and the head weights of this lane's output rows.
template <int NHG, bool FP4>
__device__ __forceinline__ void load_query(const IndexerArgs& a, int q, int n, int g, v8i* qa, int& qsc,
                                           float (*wv)[4]) {
  const uint8_t* qb = (const uint8_t*)a.qI + (int64_t)q * a.HI * kRowB<FP4>;
  qsc = 0;
#pragma unroll
  for (int hg = 0; hg < NHG; ++hg) {
    const int h = 16 * hg + n;
    const int hc = h < a.HI ? h : a.HI - 1;
    const v8i v = load_row_operand<FP4>(qb + hc * kRowB<FP4>, g);
    const int sb = (int)a.qI_scale[((int64_t)q * a.HI + hc) * 4 + g];
    const bool ok = h < a.HI;
#pragma unroll
    for (int e = 0; e < 8; ++e) qa[hg][e] = ok ? v[e] : 0;
    qsc |= (ok ? sb : 127) << (8 * hg);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hh = 16 * hg + 4 * g + i;
      const float x = a.w[(int64_t)q * a.HI + (hh < a.HI ? hh : a.HI - 1)];
      wv[hg][i] = hh < a.HI ? x : 0.f;
    }
  }
}

// Score of one page (64 entries) for one query: 4 x NHG scaled MFMAs, ReLU and head weights, then
// a reduce-scatter over the four lane groups leaves lane (n, g) with the score of slot 4n + g.
// The reduce-scatter uses the cross-half lane swaps (v_permlane32_swap: upper half of the first
// operand <-> lower half of the second; v_permlane16_swap: odd 16-lane rows of the first <-> even
// rows of the second), so the sum of the two swapped registers holds, in each half (row), the
// total of the value that half (row) keeps: three swaps and three adds, no LDS round trip.
__device__ __forceinline__ float swap_sum32(float keep_lo, float keep_hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(keep_lo), __float_as_uint(keep_hi), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap_sum16(float keep_even, float keep_odd) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(keep_even), __float_as_uint(keep_odd), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int NHG, bool FP4>
__device__ __forceinline__ float score_page(const v8i* qa, int qsc, const float (*wv)[4], const v8i* kb, int ksc) {
  v4f acc[NHG][4];
  static_for<0, NHG>::run([&](auto HGc) {
    constexpr int HG = decltype(HGc)::value;
    static_for<0, 4>::run([&](auto KGc) {
      constexpr int KG = decltype(KGc)::value;
      acc[HG][KG] = mma_scaled<HG, KG, FP4>(qa[HG], kb[KG], qsc, ksc, v4f{0.f, 0.f, 0.f, 0.f});
    });
  });
  float part[4];
#pragma unroll
  for (int kg = 0; kg < 4; ++kg) {
    float sacc = 0.f;
#pragma unroll
    for (int hg = 0; hg < NHG; ++hg)
#pragma unroll
      for (int e = 0; e < 4; ++e) sacc = fmaf(wv[hg][e], relu(acc[hg][kg][e]), sacc);
    part[kg] = sacc;
  }
  // lanes 0-31 keep key groups 0 and 1, lanes 32-63 key groups 2 and 3; then even rows keep the
  // first of the pair and odd rows the second
  const float k0 = swap_sum32(part[0], part[2]);
  const float k1 = swap_sum32(part[1], part[3]);
  return swap_sum16(k0, k1);
}

// Pages (64 entries each) scored by one wave, and page buffers in flight per wave.  Measured on the
// batched and long-context decode workloads with FP8 keys: 2 pages per wave is 15% slower than 4;
// 8 matches 4 on the first and is 4% faster on the second.
template <bool FP4>
constexpr int kPagesPerWave = FP4 ? 8 : 8;
template <bool FP4>
constexpr int kPageBufs = FP4 ? 3 : 3;
constexpr int kMaxSharedQueries = 4;   // multi-query decode: queries scored per key page

// NQ > 1 (multi-query decode): the block scores the NQ queries of one request, the last NQ tokens
// of its context, so each key page is read from HBM once for all of them instead of once per
// query.  Page buffers drop to two to make room for the extra query operands.
template <bool FP4, int NQ>
constexpr int kDecodeBufs = NQ > 1 ? 2 : kPageBufs<FP4>;

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

template <int NHG, int SEL, bool FP4, int NQ>
__global__ __launch_bounds__(256) void indexer_fp8_kernel(IndexerArgs a) {
  constexpr bool HIST = SEL == kSelHist;
  constexpr bool SK = SEL == kSelSketch && NQ == 1;
  constexpr int pages_per_wave = kPagesPerWave<FP4>;
  static_assert(!SK || pages_per_wave * kPage == kSketchSpan, "a sketch covers one wave's pages");
  constexpr int nbuf = kDecodeBufs<FP4, NQ> < pages_per_wave ? kDecodeBufs<FP4, NQ> : pages_per_wave;
  const int q0 = blockIdx.x * NQ;   // queries vary fastest: a row's blocks share one XCD (and its L2)
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
  __shared__ uint32_t lhist[HIST ? NQ : 1][HIST ? kHistBins : 1];

  const int64_t c_begin = (int64_t)blockIdx.y * 4 * pages_per_wave * kPage;
  if (c_begin >= a.max_n_vis) return;
  int r;
  int64_t nv[NQ];
  int64_t nv_max = 0;
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    nv[j] = visible_count(a, q0 + j, r);   // one request: every j gives the same r
    nv_max = nv[j] > nv_max ? nv[j] : nv_max;
  }
  // inside a fused path the selection reads only the visible prefix of each row, so a block (or
  // a wave, below) past it has nothing to do; short rows of a ragged batch then cost nothing
  if (a.visible_only && c_begin >= nv_max) return;
  if constexpr (HIST) {
    // every wave adds into every part of the histogram, so all clears must land before the first
    // add (both returns above are block-uniform, so every wave reaches this barrier)
    for (int i = tid; i < NQ * kHistBins; i += 256) lhist[i / kHistBins][i % kHistBins] = 0u;
    __syncthreads();
  }

  // A operands: the queries' indexer heads, resident in VGPRs.  Loads are unconditional (clamped
  // addresses, padded heads zeroed by select) so nothing waits before the first key page.
  v8i qa[NQ][NHG];
  int qsc[NQ];
  float wv[NQ][NHG][4];
#pragma unroll
  for (int j = 0; j < NQ; ++j) load_query<NHG, FP4>(a, q0 + j, n, g, qa[j], qsc[j], wv[j]);

  const uint8_t* keys = (const uint8_t*)a.keys;
  const int32_t* pt = a.page_table + (int64_t)(r < 0 ? 0 : r) * a.max_pages;
  const int64_t p_first = (c_begin >> 6) + (int64_t)wave * pages_per_wave;   // this wave's first page
  const int64_t vis_pages = (nv_max + kPage - 1) / kPage;

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
  auto load_page = [&](int i, v8i* kb, int& ksc) {
    int pid = __builtin_amdgcn_readlane(my_pid, i);
    pid = (unsigned)pid < (unsigned)a.num_pages ? pid : 0;
    const uint8_t* kp = keys + (int64_t)pid * (kPage * kRowB<FP4>) + 16 * lane;
    ksc = *(const int*)(a.kscale + (int64_t)pid * 256 + 4 * lane);
#pragma unroll
    for (int kg = 0; kg < 4; ++kg) kb[kg] = load_key_operand<FP4>(kp, kg);
  };

  uint32_t skey[SK ? pages_per_wave : 1];   // sketch: order key of this lane's entry of page i
  uint32_t svalid = 0u;                      // bit i: that entry is visible
  auto compute_page = [&](int i, const v8i* kb, int ksc) {
    const int64_t c0 = (p_first + i) * kPage;
    const bool mapped = page_ok(i);
    const int64_t c = c0 + 4 * n + g;
    CSA_DBG_COUNT(lane == 0 && !mapped && c0 < nv_max);   // a visible page with no page id in the pool
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      const float score = score_page<NHG, FP4>(qa[j], qsc[j], wv[j], kb, ksc);
      const float v = (mapped && c0 < nv[j] && c < nv[j]) ? score : -INFINITY;
      if (c < (a.visible_only ? nv[j] : a.max_n_vis)) {
        a.logits[(int64_t)(q0 + j) * a.ld + c] = v;
        if constexpr (HIST) {
          if (c < nv[j]) atomicAdd(&lhist[j][order_key(v) >> kHistShift], 1u);
        }
      }
      if constexpr (SK) {
        skey[i] = order_key(v);
        svalid |= (c < nv[0] ? 1u : 0u) << i;
      }
    }
  };

  // nbuf page buffers, straight-line code: the first nbuf pages are loaded up front and page
  // i + nbuf as soon as page i is scored, so up to nbuf pages are in flight and every wait is for
  // exactly the page about to be scored.  Pages past the wave's range load page 0 (always mapped)
  // and store nothing.
  if (!(a.visible_only && p_first * kPage >= nv_max)) {
    v8i kb[nbuf][4];
    int ksc[nbuf];
#pragma unroll
    for (int i = 0; i < nbuf; ++i) load_page(i, kb[i], ksc[i]);
#pragma unroll
    for (int i = 0; i < pages_per_wave; ++i) {
      compute_page(i, kb[i % nbuf], ksc[i % nbuf]);
      if (i + nbuf < pages_per_wave) load_page(i + nbuf, kb[i % nbuf], ksc[i % nbuf]);
    }
    if constexpr (SK) {
      // wave W of the row covers entries [W * kSketchSpan, (W + 1) * kSketchSpan)
      const int64_t W = p_first / pages_per_wave;
      const int64_t slot = (int64_t)q0 * a.sk_waves + W;
      sketch_wave(skey, svalid, p_first * kPage + 4 * n + g, lane, a.sk_top + slot * kSketchTop, a.sk_bound + slot);
    }
  }
  if constexpr (HIST) {
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      uint32_t* gh = a.hist + (int64_t)(q0 + j) * kHistBins;
      for (int i = tid; i < kHistBins; i += 256) {
        const uint32_t v = lhist[j][i];
        if (v) atomicAdd(&gh[i], v);
      }
    }
  }
}

// Causal prefill: every query scores the keys of request 0, so keys are shared across queries.  A
// block stages kPfPages key pages (48 KB) and their scale words in LDS once and scores kPfQueries
// consecutive queries against them (four per wave), instead of every query streaming every page.
// The staged layout is the operand order, [page][key group kg][half][lane][16 B]: lane (n, g)'s
// operand for key group kg is row 4n + kg, bytes 16g .. (half 0) and 64 + 16g .. (half 1), so every
// LDS read of an operand half is 64 lanes x 16 contiguous bytes.  Staging uses direct global-to-LDS
// loads (each lane fetches the chunk that belongs at its 16-byte slot), so no registers hold keys
// in transit.  The kernel is bound by the matrix-core / VALU pair of each page score (16 scaled
// MFMAs and 128 ReLU/weight operations), and one wave alone leaves both units half idle, so the
// block is sized for three waves per SIMD: about 160 VGPRs and 50 KB of LDS (measured on the 8192-token
// causal prefill: 8 pages at two waves per SIMD, with next-query prefetch and double-buffered key
// operands, is 18% slower).  Query blocks are issued heaviest (latest) first.  Only the visible
// prefix of each row is written: the selection reads nothing past it.
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
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3))) void indexer_fp8_prefill_kernel(
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
    v8i qa[NHG];
    int qsc;
    float wv[NHG][4];
    load_query<NHG, FP4>(a, q, n, g, qa, qsc, wv);
    for (int pi = 0; pi < np; ++pi) {
      v8i kb[4];
      const int ksc = (int)sl[pi][lane];
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
      const float score = score_page<NHG, FP4>(qa, qsc, wv, kb, ksc);
      const int64_t c = (p0 + pi) * kPage + 4 * n + g;
      if (c < a.max_n_vis) lrow[c] = (live && c < nv) ? score : -INFINITY;
    }
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
    dim3 grid((unsigned)((a.Q + kPfQueries - 1) / kPfQueries),
              (unsigned)((a.max_n_vis + kPfPages * kPage - 1) / (kPfPages * kPage)));
    ProfScope p(fp4 ? "indexer_fp4_prefill" : "indexer_fp8_prefill", s);
#define CSA_PF_LAUNCH(N)                                                                    \
  if (fp4) CSA_LAUNCH(p, (indexer_fp8_prefill_kernel<N, true>), grid, dim3(256), s, a); \
  else CSA_LAUNCH(p, (indexer_fp8_prefill_kernel<N, false>), grid, dim3(256), s, a);
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
  const int per_block = 4 * (fp4 ? kPagesPerWave<true> : kPagesPerWave<false>) * kPage;
  dim3 grid((unsigned)(a.Q / nq), (unsigned)((a.max_n_vis + per_block - 1) / per_block));
  ProfScope p(fp4 ? "indexer_fp4" : "indexer_fp8", s);
#define CSA_IDX_LAUNCH(N, F, NQ)                                                                           \
  if (hist) CSA_LAUNCH(p, (indexer_fp8_kernel<N, kSelHist, F, NQ>), grid, dim3(256), s, a);             \
  else if (sketch && NQ == 1) CSA_LAUNCH(p, (indexer_fp8_kernel<N, kSelSketch, F, 1>), grid, dim3(256), s, a); \
  else CSA_LAUNCH(p, (indexer_fp8_kernel<N, kSelNone, F, NQ>), grid, dim3(256), s, a);
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
