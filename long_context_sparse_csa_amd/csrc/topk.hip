// Per-query top-k selection over the visible prefix of each score row.
//
// Which entries are kept follows [P1] "DeepSeek-V4 全面解读" section 2.10 (top-k of the indexer
// scores, causal mask) and [P2] "DeepSeek-V4 in SGLang 深度理解分析" concept 3 (top-512; short
// contexts take every entry).  The mask is applied first, equal scores go to the lower index.
//
// Radix select on the order-preserving uint32 image of each fp32 score:
//   1. a 4096-bin histogram of the top 12 key bits (fused into the indexer at decode, or
//      topk_hist_kernel);
//   2. topk_select_kernel, many blocks per query: every block finds the threshold bin b* from the
//      histogram, appends entries above b* to the selected list and entries in b* to a candidate
//      list (wave-aggregated atomics);
//   3. the last block of each query (a done-counter with device-scope fences; no block ever waits
//      on another) resolves b* exactly: 10+10 more key bits, then, only if scores tie at the k-th
//      place, the ascending-index digits; it merges both lists and bitonic-sorts the k indices.
#include "csa_device.h"
#include "csa_internal.h"

namespace csa {

constexpr int kSelChunk = 4096;     // scores scanned per block
constexpr int kCandLds = 4096;      // candidates resolved from LDS; more fall back to global memory

__device__ __forceinline__ int64_t clamp_nv(const TopkArgs& a, int q) {
  int64_t nv = a.n_vis[q];
  return nv < 0 ? 0 : (nv > a.max_n_vis ? a.max_n_vis : nv);
}

// Exclusive prefix sum over the 256 threads of a block; *total receives the block sum.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* s_wave, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t inc = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    uint32_t t = __shfl_up(inc, off);
    if (lane >= off) inc += t;
  }
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

// Append `flag`ged values with one atomic per wave; returns this lane's slot (or -1).
__device__ __forceinline__ int64_t wave_append(bool flag, uint32_t* counter) {
  const unsigned long long m = __ballot(flag);
  if (m == 0ull) return -1;
  const int lane = threadIdx.x & 63;
  const int leader = __ffsll((long long)m) - 1;
  uint32_t base = 0;
  if (lane == leader) base = atomicAdd(counter, (uint32_t)__popcll(m));
  base = __shfl(base, leader);
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
  for (int64_t c = begin + tid; c < end; c += 256) atomicAdd(&lh[order_key(row[c]) >> kHistShift], 1u);
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

__global__ __launch_bounds__(256) void topk_select_kernel(TopkArgs a) {
  const int q = blockIdx.y, tid = threadIdx.x;
  const int64_t nv = clamp_nv(a, q);
  const int k = a.k;
  int32_t* out = a.idx + (int64_t)q * a.ld_idx;
  if (nv <= k) {
    if (blockIdx.x == 0)
      for (int i = tid; i < k; i += 256) out[i] = i < nv ? i : -1;
    return;
  }

  __shared__ uint32_t s_wave[4];
  __shared__ int s_digit;
  __shared__ uint32_t s_before, s_at;
  __shared__ int s_last;
  __shared__ uint32_t rh[2048];
  __shared__ uint2 lc[kCandLds];
  __shared__ int sk[2048];
  __shared__ uint32_t s_cursor;

  // ---- 1. threshold bin b* from the coarse histogram (descending scan, 16 bins per thread)
  const uint32_t* gh = a.hist + (int64_t)q * kHistBins;
  {
    uint32_t c[16];
    uint32_t sum = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      c[j] = gh[kHistBins - 1 - (tid * 16 + j)];
      sum += c[j];
    }
    if (tid == 0) { s_digit = -1; s_before = 0; s_at = 0; }
    __syncthreads();
    uint32_t total;
    const uint32_t pre = block_exclusive_scan(sum, s_wave, &total);
    if (pre < (uint32_t)k && pre + sum >= (uint32_t)k) {
      uint32_t acc = pre;
      for (int j = 0; j < 16; ++j) {
        if (acc + c[j] >= (uint32_t)k) {
          s_digit = kHistBins - 1 - (tid * 16 + j);
          s_before = acc;
          s_at = c[j];
          break;
        }
        acc += c[j];
      }
    }
    __syncthreads();
  }
  const int bstar = s_digit;              // -1 only if the histogram does not cover k entries
  const uint32_t above = s_before;
  const uint32_t n_b = s_at;

  // ---- 2. scan this block's chunk
  uint2* cand = a.cand + (int64_t)q * a.cand_cap;
  int32_t* sel = a.sel + (int64_t)q * k;
  uint32_t* ctr = a.counters + (int64_t)q * 4;
  const int64_t begin = (int64_t)blockIdx.x * kSelChunk;
  const int64_t end = begin + kSelChunk < nv ? begin + kSelChunk : nv;
  const float* row = a.logits + (int64_t)q * a.ld;
  if (bstar >= 0) {
    for (int64_t base = begin; base < end; base += 256) {
      const int64_t c = base + tid;
      const bool ok = c < end;
      const uint32_t key = ok ? order_key(row[c]) : 0u;
      const int bin = (int)(key >> kHistShift);
      const int64_t pa = wave_append(ok && bin > bstar, &ctr[0]);
      if (pa >= 0 && pa < (int64_t)above) sel[pa] = (int32_t)c;
      const int64_t pc = wave_append(ok && bin == bstar, &ctr[1]);
      if (pc >= 0 && pc < a.cand_cap) cand[pc] = make_uint2(key, (uint32_t)c);
    }
  }

  // ---- 3. the last block of this query finishes the selection
  __threadfence();
  __syncthreads();
  if (tid == 0) s_last = (atomicAdd(&ctr[2], 1u) == gridDim.x - 1);
  __syncthreads();
  if (!s_last) return;
  __threadfence();

  if (bstar < 0) {   // inconsistent histogram: emit an empty (all -1) selection rather than guess
    for (int i = tid; i < k; i += 256) out[i] = -1;
    return;
  }
  const uint32_t n_cand = n_b < (uint64_t)a.cand_cap ? n_b : (uint32_t)a.cand_cap;
  const bool in_lds = n_cand <= (uint32_t)kCandLds;
  if (in_lds)
    for (uint32_t i = tid; i < n_cand; i += 256) lc[i] = cand[i];
  const uint2* src = in_lds ? lc : cand;
  __syncthreads();

  // key digits: bits [19,10] then [9,0]
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

  // ties at the threshold key: keep the `need` lowest indices (3 ascending digits 11/11/10 bits)
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

  // ---- merge: entries above b* (written by every block) + resolved candidates, then sort
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

hipError_t launch_topk_hist(const TopkArgs& a, hipStream_t s) {
  if (a.max_n_vis <= a.k) return hipSuccess;
  dim3 grid((unsigned)((a.max_n_vis + kSelChunk - 1) / kSelChunk), (unsigned)a.Q);
  ProfScope p("topk_hist", s);
  hipLaunchKernelGGL(topk_hist_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_topk_select(const TopkArgs& a, hipStream_t s) {
  int64_t chunks = (a.max_n_vis + kSelChunk - 1) / kSelChunk;
  if (chunks < 1) chunks = 1;
  dim3 grid((unsigned)chunks, (unsigned)a.Q);
  ProfScope p("topk_select", s);
  hipLaunchKernelGGL(topk_select_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

// ---- preparation: clear counters/histograms, window indices, visible counts, request ids
__global__ __launch_bounds__(256) void prep_kernel(PrepArgs a) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = gid; i < a.zero_words; i += stride) a.zero_ptr[i] = 0u;
  if (a.mode == 0) return;
  for (int64_t i = gid; i < (int64_t)a.rows * kWin; i += stride) {
    const int rrow = (int)(i / kWin), j = (int)(i % kWin);
    int32_t v;
    int64_t nvis;
    if (a.mode == 1) {   // decode: ring slot of position T-128+j
      int64_t T = a.ctx_len[rrow];
      T = T < 0 ? 0 : (T > a.max_ctx ? a.max_ctx : T);
      const int64_t p = T - kWin + j;
      v = p >= 0 ? (int32_t)(p % kWin) : -1;
      nvis = T / 4;
    } else {             // causal prefill: raw position t-127+j
      const int64_t t = a.pos0 + rrow;
      const int64_t p = t - (kWin - 1) + j;
      v = p >= 0 ? (int32_t)p : -1;
      nvis = (t + 1) / 4;
    }
    a.idx[(int64_t)rrow * a.ld_idx + j] = v;
    if (j == 0) {
      a.n_vis_out[rrow] = (int32_t)nvis;
      if (a.q_req_out) a.q_req_out[rrow] = a.mode == 1 ? rrow : 0;
    }
  }
}

hipError_t launch_prep(const PrepArgs& a, hipStream_t s) {
  int64_t work = a.zero_words > (int64_t)a.rows * kWin ? a.zero_words : (int64_t)a.rows * kWin;
  int64_t blocks = (work + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 2048) blocks = 2048;
  ProfScope p("prep", s);
  hipLaunchKernelGGL(prep_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace csa
