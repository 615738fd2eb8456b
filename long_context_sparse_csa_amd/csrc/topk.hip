// Per-query top-k selection over the visible prefix of each score row.
//
// Which entries are kept follows [P1] "DeepSeek-V4 全面解读" section 2.10 (top-k of the indexer
// scores, causal mask) and [P2] "DeepSeek-V4 in SGLang 深度理解分析" concept 3 (top-512; short
// contexts take every entry).  The mask is applied first, equal scores go to the lower index.
//
// Radix select on the order-preserving uint32 image of each fp32 score:
//   1. a 4096-bin histogram of the top 12 key bits (fused into the indexer at decode, or
//      topk_hist_kernel);
//   2. topk_collect_kernel, many blocks per query: every block finds the threshold bin b* from the
//      histogram, appends entries above b* to the selected list and entries in b* to a candidate
//      list (wave-aggregated atomics);
//   3. topk_finish_kernel, one block per query, resolves b* exactly: 10+10 more key bits, then,
//      only if scores tie at the k-th place, the ascending-index digits; it emits the k indices in
//      ascending order through an LDS bitmap and a popcount scan.
// The two passes are separate launches: no block ever reads another block's plain stores within
// a launch, so no device-scope fence (an L2 write-back on this part) is needed.
#include "csa_device.h"
#include "csa_internal.h"
#include "indexer_score.h"
#include "select_block.h"

namespace csa {

constexpr int kSelChunk = 4096;     // scores scanned per block
constexpr int kCandLds = 4096;      // candidates resolved from LDS; more fall back to global memory

// Exclusive prefix sum over the 256 threads of a block; *total receives the block sum.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* s_wave, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t inc = wave_inclusive_scan(v);
  if (lane == 63) s_wave[wave] = inc;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    if (w < wave) before += s_wave[w];
    all += s_wave[w];
  }
  __syncthreads();
  *total = all;
  return before + inc - v;
}

// Append `flag`ged values with one atomic per wave (an LDS counter); returns this lane's slot or -1.
__device__ __forceinline__ int64_t wave_append(bool flag, uint32_t* counter) {
  const unsigned long long m = __ballot(flag);
  if (m == 0ull) return -1;
  const int lane = threadIdx.x & 63;
  const int leader = __ffsll((long long)m) - 1;
  uint32_t base = 0;
  if (lane == leader) base = atomicAdd(counter, (uint32_t)__popcll(m));
  base = __builtin_amdgcn_readlane(base, leader);
  if (!flag) return -1;
  const unsigned long long below = m & ((1ull << lane) - 1ull);
  return (int64_t)base + __popcll(below);
}

__global__ __launch_bounds__(256) void topk_hist_kernel(TopkArgs a) {
  const int q = blockIdx.y, tid = threadIdx.x;
  const int64_t nv = clamp_nv(a, q);
  const int64_t begin = (int64_t)blockIdx.x * kSelChunk;
  if (nv <= a.k || begin >= nv) return;
  __shared__ uint32_t lh[kHistBins];
  for (int i = tid; i < kHistBins; i += 256) lh[i] = 0u;
  __syncthreads();
  const int64_t end = begin + kSelChunk < nv ? begin + kSelChunk : nv;
  const float* row = a.logits + (int64_t)q * a.ld;
  constexpr int kPer = kSelChunk / 256;
  float vals[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int64_t c = begin + j * 256 + tid;
    vals[j] = row[c < end ? c : begin];
  }
#pragma unroll
  for (int j = 0; j < kPer; ++j)
    if (begin + j * 256 + tid < end) atomicAdd(&lh[order_key(vals[j]) >> kHistShift], 1u);
  __syncthreads();
  uint32_t* gh = a.hist + (int64_t)q * kHistBins;
  for (int i = tid; i < kHistBins; i += 256)
    if (lh[i]) atomicAdd(&gh[i], lh[i]);
}

// Find, over `nb` bins in LDS, the digit where the running count first reaches `need`.
// DESC: counting from the highest digit down; otherwise from the lowest up.  Returns the digit;
// *before = count strictly before it in scan order, *at = count of the digit itself.
template <bool DESC>
__device__ void find_digit(const uint32_t* bins, int nb, uint32_t need, uint32_t* s_wave,
                           int* s_digit, uint32_t* s_before, uint32_t* s_at) {
  const int tid = threadIdx.x;
  const int per = nb / 256;   // nb is 1024 or 2048: 4 or 8 bins per thread
  uint32_t c[8];
  uint32_t sum = 0;
  for (int j = 0; j < per; ++j) {
    const int b = DESC ? (nb - 1 - (tid * per + j)) : (tid * per + j);
    c[j] = bins[b];
    sum += c[j];
  }
  uint32_t total;
  const uint32_t pre = block_exclusive_scan(sum, s_wave, &total);
  if (pre < need && pre + sum >= need) {
    uint32_t acc = pre;
    for (int j = 0; j < per; ++j) {
      if (acc + c[j] >= need) {
        *s_digit = DESC ? (nb - 1 - (tid * per + j)) : (tid * per + j);
        *s_before = acc;
        *s_at = c[j];
        break;
      }
      acc += c[j];
    }
  }
  __syncthreads();
}

// Threshold bin b* of query q from its coarse histogram (descending scan, 16 bins per thread).
// Returns b* (or -1 when the histogram holds fewer than k entries), the count above it and in it.
__device__ void threshold_bin(const uint32_t* gh, uint32_t k, uint32_t* s_wave, int* s_digit,
                              uint32_t* s_before, uint32_t* s_at) {
  const int tid = threadIdx.x;
  uint32_t c[16];
  uint32_t sum = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    c[j] = gh[kHistBins - 1 - (tid * 16 + j)];
    sum += c[j];
  }
  if (tid == 0) { *s_digit = -1; *s_before = 0; *s_at = 0; }
  __syncthreads();
  uint32_t total;
  const uint32_t pre = block_exclusive_scan(sum, s_wave, &total);
  if (pre < k && pre + sum >= k) {
    uint32_t acc = pre;
    for (int j = 0; j < 16; ++j) {
      if (acc + c[j] >= k) {
        *s_digit = kHistBins - 1 - (tid * 16 + j);
        *s_before = acc;
        *s_at = c[j];
        break;
      }
      acc += c[j];
    }
  }
  __syncthreads();
}

// Pass 1 (many blocks per query): entries above the threshold bin go to `sel`, entries in it to
// `cand`.  Block 0 of each query records (b*, count above, count in b*) for pass 2.
__global__ __launch_bounds__(256) void topk_collect_kernel(TopkArgs a) {
  const int q = blockIdx.y, tid = threadIdx.x;
  const int64_t nv = clamp_nv(a, q);
  const int k = a.k;
  if (nv <= k) return;
  const int64_t begin = (int64_t)blockIdx.x * kSelChunk;
  if (begin >= nv && blockIdx.x != 0) return;
  __shared__ uint32_t s_wave[4];
  __shared__ int s_digit;
  __shared__ uint32_t s_before, s_at;
  // this thread's scores are loaded first (they do not depend on the threshold), so their memory
  // latency overlaps the histogram's
  const int64_t end = begin + kSelChunk < nv ? begin + kSelChunk : nv;
  const float* row = a.logits + (int64_t)q * a.ld;
  constexpr int kPer = kSelChunk / 256;
  float vals[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int64_t c = begin + j * 256 + tid;
    vals[j] = row[c < end ? c : 0];
  }
  threshold_bin(a.hist + (int64_t)q * kHistBins, (uint32_t)k, s_wave, &s_digit, &s_before, &s_at);
  const int bstar = s_digit;
  const uint32_t above = s_before;
  uint32_t* ctr = a.counters + (int64_t)q * 8;
  if (blockIdx.x == 0 && tid == 0) {
    ctr[4] = (uint32_t)bstar;
    ctr[5] = above;
    ctr[6] = s_at;
  }
  if (bstar < 0) return;
  // compact into LDS first (LDS atomics), then reserve global space with one atomic per list
  __shared__ int32_t l_above[2048];
  __shared__ uint2 l_cand[kSelChunk];
  __shared__ uint32_t s_na, s_nc, s_ga, s_gc;
  if (tid == 0) { s_na = 0u; s_nc = 0u; }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int64_t c = begin + j * 256 + tid;
    const bool ok = c < end;
    const uint32_t key = ok ? order_key(vals[j]) : 0u;
    const int bin = (int)(key >> kHistShift);
    const int64_t pa = wave_append(ok && bin > bstar, &s_na);
    if (pa >= 0 && pa < 2048) l_above[pa] = (int32_t)c;
    const int64_t pc = wave_append(ok && bin == bstar, &s_nc);
    if (pc >= 0 && pc < kSelChunk) l_cand[pc] = make_uint2(key, (uint32_t)c);
  }
  __syncthreads();
  const uint32_t na = s_na < 2048u ? s_na : 2048u, nc = s_nc < (uint32_t)kSelChunk ? s_nc : (uint32_t)kSelChunk;
  if (tid == 0) {
    s_ga = na ? atomicAdd(&ctr[0], na) : 0u;
    s_gc = nc ? atomicAdd(&ctr[1], nc) : 0u;
  }
  __syncthreads();
  uint2* cand = a.cand + (int64_t)q * a.cand_cap;
  int32_t* sel = a.sel + (int64_t)q * k;
  for (uint32_t i = tid; i < na; i += 256) {
    const uint32_t p = s_ga + i;
    if (p < above) sel[p] = l_above[i];
  }
  for (uint32_t i = tid; i < nc; i += 256) {
    const int64_t p = (int64_t)s_gc + i;
    if (p < a.cand_cap) cand[p] = l_cand[i];
  }
}

constexpr int kBitmapWords = 8192;   // ascending emission through an LDS bitmap for n_vis <= 2^18

// Pass 2 (one block per query): resolve the exact threshold inside b* (10+10 more key bits, then
// the ascending index digits only if scores tie at the k-th place) and emit the k indices in
// ascending order.
__global__ __launch_bounds__(256) void topk_finish_kernel(TopkArgs a) {
  const int q = blockIdx.x, tid = threadIdx.x;
  const int64_t nv = clamp_nv(a, q);
  const int k = a.k;
  int32_t* out = a.idx + (int64_t)q * a.ld_idx;
  if (nv <= k) {
    for (int i = tid; i < k; i += 256) out[i] = i < nv ? i : -1;
    return;
  }
  __shared__ uint32_t s_wave[4];
  __shared__ int s_digit;
  __shared__ uint32_t s_before, s_at, s_cursor;
  __shared__ uint32_t rh[2048];
  __shared__ uint2 lc[kCandLds];
  __shared__ __align__(16) uint32_t bm[kBitmapWords];     // bitmap, or (n_vis > 2^18) the sort buffer
  __shared__ __align__(16) uint32_t pf[kBitmapWords];   // exclusive prefix count of each bitmap word
  const uint32_t* ctr = a.counters + (int64_t)q * 8;
  const uint2* cand = a.cand + (int64_t)q * a.cand_cap;
  const int32_t* sel = a.sel + (int64_t)q * k;
  // the candidate list (up to what LDS holds) and the entries above b* are loaded together with
  // the counters, before their counts are known (addresses clamped to the buffers), so the block
  // waits for one memory round trip instead of two
  constexpr int kPer = kCandLds / 256;
  uint2 tmp[kPer];
  {
    const int64_t cap = a.cand_cap < kCandLds ? a.cand_cap : kCandLds;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int64_t i = j * 256 + tid;
      tmp[j] = cand[i < cap ? i : cap - 1];
    }
  }
  int32_t cs[8];   // above < k <= 2048: at most 8 per thread
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int i = j * 256 + tid;
    cs[j] = sel[i < k ? i : k - 1];
  }
  const int bstar = (int)ctr[4];
  const uint32_t above = ctr[5];
  const uint32_t n_b = ctr[6];
  if (bstar < 0) {   // inconsistent histogram: emit an empty (all -1) selection rather than guess
    for (int i = tid; i < k; i += 256) out[i] = -1;
    return;
  }
  const uint32_t n_cand = n_b < (uint64_t)a.cand_cap ? n_b : (uint32_t)a.cand_cap;
  const bool in_lds = n_cand <= (uint32_t)kCandLds;
  if (in_lds) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const uint32_t i = j * 256 + tid;
      if (i < n_cand) lc[i] = tmp[j];
    }
  }
  const uint2* src = in_lds ? lc : cand;
  __syncthreads();

  uint32_t prefix = (uint32_t)bstar;
  int pbits = 12;
  uint32_t need = (uint32_t)k - above;
  uint32_t eq_at = n_cand;
  for (int pass = 0; pass < 2; ++pass) {
    for (int i = tid; i < 1024; i += 256) rh[i] = 0u;
    __syncthreads();
    const int shift = 32 - pbits - 10;
    for (uint32_t i = tid; i < n_cand; i += 256) {
      const uint32_t key = src[i].x;
      if ((key >> (32 - pbits)) == prefix) atomicAdd(&rh[(key >> shift) & 1023u], 1u);
    }
    __syncthreads();
    if (tid == 0) { s_digit = 0; s_before = 0; s_at = 0; }
    __syncthreads();
    find_digit<true>(rh, 1024, need, s_wave, &s_digit, &s_before, &s_at);
    prefix = (prefix << 10) | (uint32_t)s_digit;
    pbits += 10;
    need -= s_before;
    eq_at = s_at;
  }
  const uint32_t T = prefix;

  uint32_t idx_thr = 0xFFFFFFFFu;
  if (need < eq_at) {
    uint32_t ipre = 0;
    int ibits = 0;
    const int widths[3] = {11, 11, 10};
    for (int pass = 0; pass < 3; ++pass) {
      const int wdt = widths[pass];
      for (int i = tid; i < 2048; i += 256) rh[i] = 0u;
      __syncthreads();
      const int shift = 32 - ibits - wdt;
      for (uint32_t i = tid; i < n_cand; i += 256) {
        const uint2 x = src[i];
        if (x.x == T && (ibits == 0 || (x.y >> (32 - ibits)) == ipre))
          atomicAdd(&rh[(x.y >> shift) & ((1u << wdt) - 1u)], 1u);
      }
      __syncthreads();
      if (tid == 0) { s_digit = 0; s_before = 0; s_at = 0; }
      __syncthreads();
      find_digit<false>(rh, 2048, need, s_wave, &s_digit, &s_before, &s_at);
      ipre = (ipre << wdt) | (uint32_t)s_digit;
      ibits += wdt;
      need -= s_before;
    }
    idx_thr = ipre;
  }

  if (nv <= (int64_t)kBitmapWords * 32) {
    // ascending emission: set one bit per selected index, then a block-wide popcount scan
    const int words = (int)((nv + 31) / 32);
    for (int i = tid; i < words; i += 256) bm[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j * 256 + tid < (int)above) atomicOr(&bm[cs[j] >> 5], 1u << (cs[j] & 31));
    for (uint32_t i = tid; i < n_cand; i += 256) {
      const uint2 x = src[i];
      if (x.x > T || (x.x == T && x.y <= idx_thr)) atomicOr(&bm[x.y >> 5], 1u << (x.y & 31));
    }
    __syncthreads();
    // rank placement: thread t owns words [32t, 32t+32) and writes each word's exclusive prefix
    // count to pf; then every selected index lands at pf[word] + the set bits below it in its
    // word.  No per-bit loops: a loop over each lane's bits measured 5 us on the long rows.
    static_assert(kBitmapWords == 256 * 32, "256 threads of 32 words cover the bitmap");
    uint32_t wb[32];
#pragma unroll
    for (int j = 0; j < 32; j += 4) {
      const uint4 v = *(const uint4*)&bm[32 * tid + j];   // words past `words` were never cleared
      wb[j] = 32 * tid + j < words ? v.x : 0u;
      wb[j + 1] = 32 * tid + j + 1 < words ? v.y : 0u;
      wb[j + 2] = 32 * tid + j + 2 < words ? v.z : 0u;
      wb[j + 3] = 32 * tid + j + 3 < words ? v.w : 0u;
    }
    uint32_t cnt = 0;
#pragma unroll
    for (int j = 0; j < 32; ++j) cnt += __popc(wb[j]);
    uint32_t total;
    uint32_t run = block_exclusive_scan(cnt, s_wave, &total);
#pragma unroll
    for (int j = 0; j < 32; j += 4) {
      uint32_t p4[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        p4[u] = run;
        run += __popc(wb[j + u]);
      }
      *(uint4*)&pf[32 * tid + j] = make_uint4(p4[0], p4[1], p4[2], p4[3]);
    }
    __syncthreads();
    // positions are staged in LDS (the radix bins are free by now; k <= 2048 fits) and stored to
    // the output in one coalesced pass
    int32_t* stage = (int32_t*)rh;
    auto place = [&](uint32_t i) {
      const uint32_t pos = pf[i >> 5] + __popc(bm[i >> 5] & ((1u << (i & 31)) - 1u));
      if (pos < (uint32_t)k) stage[pos] = (int32_t)i;
    };
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j * 256 + tid < (int)above) place((uint32_t)cs[j]);
    for (uint32_t i = tid; i < n_cand; i += 256) {
      const uint2 x = src[i];
      if (x.x > T || (x.x == T && x.y <= idx_thr)) place(x.y);
    }
    __syncthreads();
    for (int i = tid; i < k; i += 256) out[i] = i < (int)total ? stage[i] : -1;   // -1: short histogram
    return;
  }

  // n_vis > 2^18: merge into the sort buffer and bitonic-sort the k indices
  int* sk = (int*)bm;
  int K2 = 1;
  while (K2 < k) K2 <<= 1;
  for (int i = tid; i < K2; i += 256) sk[i] = (i < (int)above) ? sel[i] : 0x7FFFFFFF;
  if (tid == 0) s_cursor = 0u;
  __syncthreads();
  for (uint32_t i = tid; i < n_cand; i += 256) {
    const uint2 x = src[i];
    if (x.x > T || (x.x == T && x.y <= idx_thr)) {
      const uint32_t p = atomicAdd(&s_cursor, 1u);
      if (above + p < (uint32_t)k) sk[above + p] = (int)x.y;
    }
  }
  __syncthreads();
  for (int size = 2; size <= K2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < K2 / 2; i += 256) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool asc = (lo & size) == 0;
        const int x = sk[lo], y = sk[hi];
        if ((x > y) == asc) { sk[lo] = y; sk[hi] = x; }
      }
      __syncthreads();
    }
  }
  for (int i = tid; i < k; i += 256) out[i] = sk[i] == 0x7FFFFFFF ? -1 : sk[i];
}

// NT threads cover rows of up to NT * PER entries; short rows take a small block so that several
// rows share a CU.
template <int NT, int PER>
__global__ __launch_bounds__(NT) void topk_single_kernel(TopkArgs a) {
  constexpr int kRowMax = NT * PER;
  const int q = blockIdx.x, tid = threadIdx.x;
  const int k = a.k;
  int32_t* out = a.idx + (int64_t)q * a.ld_idx;
  // the row's extent word and the request's page ids are loaded together (one wait), then the
  // scores up to the row's length: two memory round trips before the first barrier, not three
  const int32_t word = row_extent_word(a, q);
  const int r = a.win_mode == 1 ? q / a.q_per_req : 0;   // request of this query (prefill: 0)
  const int32_t* pt = a.rows ? a.page_table + (int64_t)r * a.max_pages : nullptr;
  static_assert(kRowMax / kPage <= NT, "one page id per thread");
  const int n_pt = a.rows ? (a.max_pages < kRowMax / kPage ? a.max_pages : kRowMax / kPage) : 0;
  const int32_t pg_mine = tid < n_pt ? pt[tid] : -1;
  int64_t seen;
  const int64_t nv = row_extent(a, q, word, seen);
  if (a.win_mode) write_window(a, q, seen);
  auto row_of = [&](int c, int pg) { return (unsigned)pg < (unsigned)a.num_pages ? pg * kPage + (c & (kPage - 1)) : -1; };
  __shared__ int32_t pt_lds[kRowMax / kPage];
  __shared__ SelShared<NT> sh;

  const float* row = a.logits + (int64_t)q * a.ld;
  const int c0 = tid * PER;          // this thread owns entries [c0, c0+PER)
  uint32_t key[PER];
  uint32_t vm = 0;
  if (nv > k) {
    float v[PER];
#pragma unroll
    for (int j = 0; j < PER; j += 4) {
      const int c = c0 + j;
      // rows are 16-byte aligned and ld is a multiple of 4; entries past n_vis are never counted
      const float4 x = *(const float4*)(row + (c < nv ? c : 0));
      v[j] = x.x; v[j + 1] = x.y; v[j + 2] = x.z; v[j + 3] = x.w;
    }
    // after the score loads in program order: the store waits for its page id, and the compiler
    // keeps LDS stores and the scores' loads in order
    if (tid < n_pt) pt_lds[tid] = pg_mine;
    // cleared while the loads are in flight
    for (int i = tid; i < kHistBins; i += NT) sh.bins[i] = 0u;
    if (tid == 0) sh.s_ncand = 0u;
#pragma unroll
    for (int j = 0; j < PER; ++j) key[j] = order_key_raw(v[j]);
    vm = prefix_mask<PER>(c0, nv);
    publish_extremes<NT, PER>(key, vm, sh);   // read after the barrier below
  } else if (tid < n_pt) {
    pt_lds[tid] = pg_mine;
  }
  __syncthreads();
  if (nv <= k) {   // block-uniform
    for (int i = tid; i < k; i += NT) {
      out[i] = i < nv ? i : -1;
      if (a.rows) a.rows[(int64_t)q * a.ld_rows + i] = i < nv ? row_of(i, pt_lds[i >> 6]) : -1;
    }
    return;
  }
  block_threshold<NT, PER, true, true>(key, vm, (uint32_t)k, sh);
  block_emit<NT, PER>(key, vm, sh.s_T, sh.s_need, (uint32_t)k, [&](int j) { return c0 + j; }, sh);
  const int32_t* sel = (const int32_t*)sh.cand_sel;
  for (int i = tid; i < k; i += NT) {
    const int c = sel[i];
    out[i] = c;
    if (a.rows) {
      const int rw = row_of(c, pt_lds[c >> 6]);
      CSA_DBG_COUNT(rw < 0);   // a selected entry on a page with no page id in the pool
      a.rows[(int64_t)q * a.ld_rows + i] = rw;
    }
  }
}

// ---- long decode rows: selection from the indexer's per-wave sketches.  Wave W of a row (entries
// [512 W, 512 W + 512)) left its 8 largest scores (ascending indices) and a bound on the rest, so
// the sketches of a 262,144-entry row are 4,096 entries in index order.  One block of 1024
// threads finds their exact k-th largest key T as the short-row selection does.  If every wave's
// bound lies below T, no entry left out of the sketches can reach T and the sketches' top k is the
// row's; otherwise (ties at T, or a wave holding more than 8 of the row's top entries) the block
// selects from the full score row instead (select_streamed).

template <int PER>
__global__ __launch_bounds__(1024) void topk_sketch_kernel(TopkArgs a) {
  constexpr int NT = 1024;
  const int q = blockIdx.x, tid = threadIdx.x;
  const int k = a.k;
  int32_t* out = a.idx + (int64_t)q * a.ld_idx;
  int32_t* rows_out = a.rows ? a.rows + (int64_t)q * a.ld_rows : nullptr;
  // the row's extent word, its sketch entries and its wave bounds (over the whole sketch row: in
  // bounds, masked once the row's length is known) are loaded together, before the first wait
  const int32_t word = row_extent_word(a, q);
  const uint2* top = a.sk_top + (int64_t)q * a.sk_waves * kSketchTop;
  const uint32_t* bound = a.sk_bound + (int64_t)q * a.sk_waves;
  const int64_t n_u_max = a.sk_waves * kSketchTop;
  uint32_t key[PER];
  uint32_t idx[PER];
  const int64_t u0 = (int64_t)tid * PER;            // this thread's sketch entries [u0, u0 + PER)
#pragma unroll
  for (int j = 0; j < PER; j += 2) {
    const int64_t u = u0 + j;
    const uint4 x = *(const uint4*)&top[u < n_u_max ? u : 0];   // two entries; rows hold multiples of 8
    key[j] = x.x; idx[j] = x.y; key[j + 1] = x.z; idx[j + 1] = x.w;
  }
  uint32_t bnd[(kSketchMaxWaves + NT - 1) / NT];
#pragma unroll
  for (int i = 0; i < (kSketchMaxWaves + NT - 1) / NT; ++i) {
    const int64_t W = tid + (int64_t)i * NT;
    bnd[i] = W < a.sk_waves ? bound[W] : 0u;
  }
  int64_t seen;
  const int64_t nv = row_extent(a, q, word, seen);
  if (a.win_mode) write_window(a, q, seen);
  const int r = q / a.q_per_req;
  const int32_t* pt = a.page_table + (int64_t)r * a.max_pages;
  auto row_of = [&](int c) {
    const int pg = pt[c >> 6];
    return (unsigned)pg < (unsigned)a.num_pages ? pg * kPage + (c & (kPage - 1)) : -1;
  };
  if (nv <= k) {
    for (int i = tid; i < k; i += NT) {
      out[i] = i < nv ? i : -1;
      if (rows_out) rows_out[i] = i < nv ? row_of(i) : -1;
    }
    return;
  }
  __shared__ SelShared<NT> sh;
  const int64_t n_w = (nv + kSketchSpan - 1) / kSketchSpan;
  const int64_t n_u = n_w * kSketchTop;               // sketch entries of the row (<= NT * PER)
  uint32_t vm = 0u;
#pragma unroll
  for (int i = 0; i < (kSketchMaxWaves + NT - 1) / NT; ++i) bnd[i] = tid + (int64_t)i * NT < n_w ? bnd[i] : 0u;
  for (int i = tid; i < kHistBins; i += NT) sh.bins[i] = 0u;
  if (tid == 0) sh.s_ncand = 0u;
#pragma unroll
  for (int j = 0; j < PER; ++j) vm |= (u0 + j < n_u && idx[j] != 0xFFFFFFFFu ? 1u : 0u) << j;
  {
    const uint32_t wsum = wave_inclusive_scan(__popc(vm));   // lane 63 holds the wave's count
    if ((tid & 63) == 63) sh.scan[tid >> 6] = wsum;
  }
  __syncthreads();
  uint32_t n_real = 0u;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) n_real += sh.scan[w];
  // a row whose sketches hold fewer than k entries is selected from its full scores
  bool from_sketch = n_real >= (uint32_t)k;
  if (from_sketch) {
    block_threshold<NT, PER>(key, vm, (uint32_t)k, sh);
    const uint32_t T = sh.s_T;
    bool reach = false;
#pragma unroll
    for (int i = 0; i < (kSketchMaxWaves + NT - 1) / NT; ++i) reach |= tid + (int64_t)i * NT < n_w && bnd[i] >= T;
    from_sketch = !__syncthreads_or(reach);
  }
  if (from_sketch) {
    block_emit<NT, PER>(key, vm, sh.s_T, sh.s_need, (uint32_t)k, [&](int j) { return (int32_t)idx[j]; }, sh);
    const int32_t* sel = (const int32_t*)sh.cand_sel;
    for (int i = tid; i < k; i += NT) {
      const int c = sel[i];
      out[i] = c;
      if (rows_out) {
        const int rw = row_of(c);
        CSA_DBG_COUNT(rw < 0);
        rows_out[i] = rw;
      }
    }
    return;
  }
  if (a.ia.sk_rescore_from > 0 && nv >= a.ia.sk_rescore_from) {
    // the indexer stored no scores for this row: rescore it, each wave a span at a time
    const int wave = tid >> 6, lane = tid & 63;
    const int64_t n_span = (nv + kSketchSpan - 1) / kSketchSpan;
    const int nhg = (a.ia.HI + 15) / 16;
    for (int64_t W = wave; W < n_span; W += NT / 64) {
      if (a.ia.dt == 3) {
        switch (nhg) {
          case 1: rescore_span<1, true>(a.ia, q, W, lane); break;
          case 2: rescore_span<2, true>(a.ia, q, W, lane); break;
          case 3: rescore_span<3, true>(a.ia, q, W, lane); break;
          default: rescore_span<4, true>(a.ia, q, W, lane); break;
        }
      } else {
        switch (nhg) {
          case 1: rescore_span<1, false>(a.ia, q, W, lane); break;
          case 2: rescore_span<2, false>(a.ia, q, W, lane); break;
          case 3: rescore_span<3, false>(a.ia, q, W, lane); break;
          default: rescore_span<4, false>(a.ia, q, W, lane); break;
        }
      }
    }
    __syncthreads();   // the block reads the rescored row next (workgroup scope: one L1)
  }
  select_streamed<NT>(a, q, nv, (uint32_t)k, sh, out, rows_out, pt);
}

hipError_t launch_topk_single(const TopkArgs& a, hipStream_t s) {
  ProfScope p("topk_single", s);
  if (a.max_n_vis <= 128 * kSinglePer)
    CSA_LAUNCH(p, (topk_single_kernel<128, kSinglePer>), dim3((unsigned)a.Q), dim3(128), s, a);
  else if (a.max_n_vis <= 256 * kSinglePer)
    CSA_LAUNCH(p, (topk_single_kernel<256, kSinglePer>), dim3((unsigned)a.Q), dim3(256), s, a);
  else if (a.max_n_vis <= 1024 * kSinglePer)
    CSA_LAUNCH(p, (topk_single_kernel<1024, kSinglePer>), dim3((unsigned)a.Q), dim3(1024), s, a);
  else
    CSA_LAUNCH(p, (topk_single_kernel<1024, 32>), dim3((unsigned)a.Q), dim3(1024), s, a);
  return hipGetLastError();
}

hipError_t launch_topk_sketch(const TopkArgs& a, hipStream_t s) {
  const int64_t entries = topk_sketch_waves(a.max_n_vis) * kSketchTop;
  ProfScope p("topk_sketch", s);
  if (entries <= 1024 * 4) CSA_LAUNCH(p, (topk_sketch_kernel<4>), dim3((unsigned)a.Q), dim3(1024), s, a);
  else if (entries <= 1024 * 8) CSA_LAUNCH(p, (topk_sketch_kernel<8>), dim3((unsigned)a.Q), dim3(1024), s, a);
  else CSA_LAUNCH(p, (topk_sketch_kernel<16>), dim3((unsigned)a.Q), dim3(1024), s, a);
  return hipGetLastError();
}

hipError_t launch_topk_hist(const TopkArgs& a, hipStream_t s) {
  if (a.max_n_vis <= a.k) return hipSuccess;
  dim3 grid((unsigned)((a.max_n_vis + kSelChunk - 1) / kSelChunk), (unsigned)a.Q);
  ProfScope p("topk_hist", s);
  CSA_LAUNCH(p, topk_hist_kernel, grid, dim3(256), s, a);
  return hipGetLastError();
}

hipError_t launch_topk_select(const TopkArgs& a, hipStream_t s) {
  int64_t chunks = (a.max_n_vis + kSelChunk - 1) / kSelChunk;
  if (chunks < 1) chunks = 1;
  if (a.max_n_vis > a.k) {
    ProfScope p("topk_collect", s);
    CSA_LAUNCH(p, topk_collect_kernel, dim3((unsigned)chunks, (unsigned)a.Q), dim3(256), s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  ProfScope p("topk_finish", s);
  CSA_LAUNCH(p, topk_finish_kernel, dim3((unsigned)a.Q), dim3(256), s, a);
  return hipGetLastError();
}

// ---- preparation: clear counters/histograms, window indices, visible counts, request ids, and
// (layers without an indexer) the dense compressed index lists
// visible compressed entries of row rrow: every entry whose `ratio` raw tokens are all at or before
// the row's position (decode: T tokens, the current one included; prefill: position t)
__device__ __forceinline__ int64_t prep_visible(const PrepArgs& a, int rrow) {
  if (a.mode == 1) {
    int r;
    return decode_seen(a.ctx_len, a.max_ctx, a.q_per_req, rrow, r) / a.ratio;
  }
  return (a.pos0 + rrow + 1) / a.ratio;
}

__global__ __launch_bounds__(256) void prep_kernel(PrepArgs a) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = gid; i < a.zero_words; i += stride) a.zero_ptr[i] = 0u;
  if (a.mode == 0) return;
  for (int64_t i = gid; i < (int64_t)a.rows * kWin; i += stride) {
    const int rrow = (int)(i / kWin), j = (int)(i % kWin);
    int32_t v;
    if (a.mode == 1) {   // decode: ring slot of the j-th of the 128 positions up to the row's
      int r;
      const int64_t p = decode_seen(a.ctx_len, a.max_ctx, a.q_per_req, rrow, r) - kWin + j;
      v = p >= 0 ? ring_slot(p, a.ring) : -1;
    } else {             // causal prefill: raw position t-127+j
      const int64_t t = a.pos0 + rrow;
      const int64_t p = t - (kWin - 1) + j;
      v = p >= 0 ? (int32_t)p : -1;
    }
    a.idx[(int64_t)rrow * a.ld_idx + j] = v;
    if (j == 0) {
      a.n_vis_out[rrow] = (int32_t)prep_visible(a, rrow);
      if (a.q_req_out) a.q_req_out[rrow] = a.mode == 1 ? rrow / a.q_per_req : 0;
    }
  }
  // dense compressed list: entry j while visible, then -1 (row-major, so stores coalesce)
  for (int64_t i = gid; i < (int64_t)a.rows * a.comp_cols; i += stride) {
    const int rrow = (int)(i / a.comp_cols);
    const int64_t j = i % a.comp_cols;
    a.idx[(int64_t)rrow * a.ld_idx + kWin + j] = j < prep_visible(a, rrow) ? (int32_t)j : -1;
  }
}

hipError_t launch_prep(const PrepArgs& a, hipStream_t s) {
  int64_t work = a.zero_words > (int64_t)a.rows * kWin ? a.zero_words : (int64_t)a.rows * kWin;
  if ((int64_t)a.rows * a.comp_cols > work) work = (int64_t)a.rows * a.comp_cols;
  int64_t blocks = (work + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 2048) blocks = 2048;
  ProfScope p("prep", s);
  CSA_LAUNCH(p, prep_kernel, dim3((unsigned)blocks), dim3(256), s, a);
  return hipGetLastError();
}

CSA_DBG_ACCESSOR(debug_take_violations_topk)

}  // namespace csa
