// One-block exact top-k selection and the row helpers shared by the selection kernels
// (topk.hip) and the decode attention that selects its own rows (attention.hip).
//
// Which entries are kept follows [P1] "DeepSeek-V4 全面解读" section 2.10 (top-k of the indexer
// scores, causal mask) and [P2] "DeepSeek-V4 in SGLang 深度理解分析" concept 3 (top-512; short
// contexts take every entry); equal scores go to the lower index.
#pragma once
#include "csa_device.h"
#include "csa_internal.h"

namespace csa {

__device__ __forceinline__ int64_t clamp_nv(const TopkArgs& a, int q) {
  int64_t nv = a.n_vis[q];
  return nv < 0 ? 0 : (nv > a.max_n_vis ? a.max_n_vis : nv);
}

// The one word of memory row q's extent depends on: its request's context length (decode), its
// n_vis entry, or none (causal prefill).  The selection prologues issue it with their other loads
// and resolve the extent after one wait, instead of a chain of dependent loads.
__device__ __forceinline__ int32_t row_extent_word(const TopkArgs& a, int q) {
  return a.win_mode == 1 ? a.ctx_len[q / a.q_per_req] : (a.win_mode == 2 ? 0 : a.n_vis[q]);
}

// Visible count of row q from that word (decode: tokens seen / 4, prefill: (t+1)/4, else n_vis),
// clamped to [0, max_n_vis]; `seen` gets the decode query's tokens seen (0 otherwise).
__device__ __forceinline__ int64_t row_extent(const TopkArgs& a, int q, int32_t word, int64_t& seen) {
  int64_t nv;
  seen = 0;
  if (a.win_mode == 1) {
    seen = decode_seen_of(word, a.max_ctx, a.q_per_req, q);
    nv = seen / 4;
  } else if (a.win_mode == 2) {
    nv = (a.pos0 + q + 1) / 4;
  } else {
    nv = word;
  }
  return nv < 0 ? 0 : (nv > a.max_n_vis ? a.max_n_vis : nv);
}

__device__ __forceinline__ int64_t topk_row_count(const TopkArgs& a, int q) {
  int64_t seen;
  return row_extent(a, q, row_extent_word(a, q), seen);
}

// Window part of the index list: decode ring slots (position % ring) of the 128 positions up to
// the query's (`seen` from row_extent), or prefill positions t-127..t; -1 before position 0.
// Written to columns [-128, 0) relative to a.idx.
__device__ __forceinline__ void write_window(const TopkArgs& a, int q, int64_t seen) {
  const int j = threadIdx.x;
  if (j >= kWin) return;
  int32_t v;
  if (a.win_mode == 1) {
    const int64_t p = seen - kWin + j;
    v = p >= 0 ? ring_slot(p, a.ring) : -1;
  } else {
    const int64_t p = a.pos0 + q - (kWin - 1) + j;
    v = p >= 0 ? (int32_t)p : -1;
  }
  a.idx[(int64_t)q * a.ld_idx - kWin + j] = v;
}


// ---- single-block selection: one block per query keeps its entries in registers (PER consecutive
// entries per thread, in index order), so no global histogram, no zeroed workspace and no second
// launch are needed.  Two users: short rows (n_vis <= kSingleMax), whose entries are the row itself,
// and long decode rows, whose entries are the indexer's per-wave sketches (see topk_sketch_kernel).
// Every barrier-separated phase costs on the order of a microsecond at 16 waves, and a predicated
// LDS instruction costs its issue slot even when few lanes are active, so the phases are few, the
// scans are done by a single wave and sparse passes skip instructions no lane needs:
//   1. a 4096-bin histogram of the scores over the entries' value range gives the threshold bin b*
//      and the count above it; b*'s entries (normally a handful) go to an LDS candidate list and
//      one wave ranks them by their full keys, giving the exact k-th largest key T and how many
//      keys equal to T are taken;
//   2. when b* holds more than 64 entries (ties, clusters) or a score is not finite, the levels run
//      on key prefixes instead: a 12-bit histogram of every key gives b*, and the keys of its
//      entries are resolved by one wave (two 10-bit levels of the remaining 20 bits, no block
//      barrier), or by two block-wide levels when more than kCandMax entries share b*;
//   3. one block scan of the per-thread (greater, equal) counts, packed in one word, places the k
//      indices in ascending order (equal keys at T in index order) in LDS, from where they are
//      written with coalesced stores.
constexpr int kSinglePer = 16;      // entries per thread, in index order (32 for the longest rows)
constexpr int kCandMax = 2048;      // entries of the threshold bin resolved by one wave; more take
                                    // the block-wide path

// One wave scans `nb` bins (64 to 4096, a multiple of 256) from the top and finds the bin where
// the running count first reaches `need` (1 <= need <= total): *digit, *before (count strictly
// above it).  Two rounds, no serial search: per-lane sums and a shuffle scan pick the lane whose
// range crosses `need`, then the 64 lanes read that range's bins one each and a second scan picks
// the bin.  Lanes of other waves do nothing; the caller puts barriers around it.
__device__ __forceinline__ void wave_find_desc(const uint32_t* bins, int nb, uint32_t need, uint32_t* digit,
                                               uint32_t* before) {
  const int lane = threadIdx.x & 63;
  const int per = nb / 64;              // bins per lane: lane l owns [nb - per (l+1), nb - per l)
  const int hi = nb - per * lane;       // exclusive top of this lane's range
  uint32_t sum = 0;
  for (int j = 0; j < per; j += 4) {
    const uint4 c = *(const uint4*)&bins[hi - per + j];
    sum += c.x + c.y + c.z + c.w;
  }
  const uint32_t inc = wave_inclusive_scan(sum);
  const uint64_t cross = __ballot(inc - sum < need && inc >= need);
  const int x = cross ? __ffsll((long long)cross) - 1 : 63;
  const uint32_t pre_x = __builtin_amdgcn_readlane(inc - sum, x);
  const int top = nb - per * x;         // lane j looks at bin top - 1 - j
  const uint32_t c = lane < per ? bins[top - 1 - lane] : 0u;
  const uint32_t cinc = wave_inclusive_scan(c);
  const uint64_t hit = __ballot(lane < per && pre_x + cinc >= need);
  const int y = hit ? __ffsll((long long)hit) - 1 : 0;
  if (lane == y) {
    *digit = (uint32_t)(top - 1 - y);
    *before = pre_x + cinc - c;
  }
}

// the score of an order key (the inverse of order_key; -0.0 comes back as +0.0)
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// LDS of the one-block selection (16 KB of bins + 8 KB of candidate keys / selected indices).
template <int NT>
struct SelShared {
  uint32_t bins[kHistBins];
  uint32_t scan[NT / 64];          // per-wave totals of the final scan
  // order keys of the threshold bin's entries while the threshold is resolved, then the selected
  // indices
  uint32_t cand_sel[kCandMax > kSingleMaxK ? kCandMax : kSingleMaxK];
  uint32_t s_digit, s_before, s_ncand, s_T, s_need;
  uint32_t s_all_eq;               // 1: every real entry equal to T is taken (the k are those >= T)
  uint32_t ext[2 * (NT / 64)];     // per-wave largest / smallest key
};

// Exact k-th largest order key T among the block's entries (thread t holds key[0..PER) with bit j
// of vm set for a real entry) and how many entries equal to T are taken: sh.s_T, sh.s_need on
// return (after a barrier).  The block holds at least k real entries.  On entry sh.bins is zeroed,
// sh.s_ncand is 0 and a barrier has passed since.
// All PER entries of a thread real: the per-entry validity tests drop out (every thread but the
// last of a row takes these paths, so the VALU work per entry, which bounds each phase, shrinks).
template <int PER>
__device__ __forceinline__ bool all_real(uint32_t vm) {
  return vm == (PER >= 32 ? 0xFFFFFFFFu : ((1u << PER) - 1u));
}

// vm of a thread whose entries [c0, c0 + PER) are real below n: a prefix of them
template <int PER>
__device__ __forceinline__ uint32_t prefix_mask(int64_t c0, int64_t n) {
  const int64_t m = n - c0;
  return m >= PER ? (PER >= 32 ? 0xFFFFFFFFu : ((1u << PER) - 1u)) : (m <= 0 ? 0u : ((1u << (uint32_t)m) - 1u));
}

// The extremes of the block's real keys, per wave into sh.ext (largest, then smallest), visible after
// the caller's next barrier.  A caller that publishes them with its own keys' barrier saves
// block_threshold a pass and a barrier (EXT = true).
template <int NT, int PER>
__device__ __forceinline__ void publish_extremes(const uint32_t* key, uint32_t vm, SelShared<NT>& sh) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  uint32_t kmx = 0u, kmn = 0xFFFFFFFFu;
  if (all_real<PER>(vm)) {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      kmx = key[j] > kmx ? key[j] : kmx;
      kmn = key[j] < kmn ? key[j] : kmn;
    }
  } else {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      if ((vm >> j) & 1u) {
        kmx = key[j] > kmx ? key[j] : kmx;
        kmn = key[j] < kmn ? key[j] : kmn;
      }
    }
  }
  kmx = wave_umax(kmx);
  kmn = ~wave_umax(~kmn);   // min through the max of complements
  if (lane == 0) {
    sh.ext[wave] = kmx;
    sh.ext[NT / 64 + wave] = kmn;
  }
}

// RAW: the keys come from order_key_raw; the key-prefix levels then first map NaNs to 0 in place
// (the value-range level never runs on rows with a non-finite key, and its bins only need a
// monotone function of the key).  EXT: the caller published the extremes (publish_extremes) before
// the barrier that precedes this call.
template <int NT, int PER, bool RAW = false, bool EXT = false>
__device__ void block_threshold(uint32_t* key, uint32_t vm, uint32_t k, SelShared<NT>& sh) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const bool full = all_real<PER>(vm);
  if constexpr (!EXT) {
    publish_extremes<NT, PER>(key, vm, sh);
    __syncthreads();
  }
  // Level 1 on the value range: 4096 equal-width bins between the smallest and largest finite
  // score.  Scores crowd a few of the fixed 12-bit key-prefix bins (the exponent and three
  // mantissa bits), so LDS atomics collide and the threshold bin holds hundreds of entries; on the
  // value range the bins hold a handful.  The bin index is a monotone function of the score (one
  // fused multiply-add with a positive scale, a clamp and truncation all preserve order) applied
  // to every entry alike, so b* and the counts above it are exact.  When b* holds at most 64 entries one wave ranks them by
  // their full keys; otherwise (ties, clusters, non-finite scores) the key-prefix levels run.
  bool resolved = false;
  {
    uint32_t kmax = 0u, kmin = 0xFFFFFFFFu;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
      kmax = sh.ext[w] > kmax ? sh.ext[w] : kmax;
      kmin = sh.ext[NT / 64 + w] < kmin ? sh.ext[NT / 64 + w] : kmin;
    }
    const float vmin = key_value(kmin), vmax = key_value(kmax);
    const float scale = 4096.f / (vmax - vmin);
    // every real key is finite (NaN keys lie below -inf's, raw ones also above +inf's; infinities
    // outside +-FLT_MAX) and spread
    const uint32_t kfin_lo = RAW ? order_key_raw(-3.40282347e+38f) : order_key(-3.40282347e+38f);
    const uint32_t kfin_hi = RAW ? order_key_raw(3.40282347e+38f) : order_key(3.40282347e+38f);
    const bool adaptive = kmin >= kfin_lo && kmax <= kfin_hi &&
                          kmax > kmin && scale > 0.f && scale < 3.0e38f;
    if (adaptive) {
      uint32_t bin[PER];
      const float off = -vmin * scale;
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        // about 0 at vmin and 4096 at vmax (finite for real entries; the others, never counted,
        // are clamped too)
        const float x = fmaf(key_value(key[j]), scale, off);
        const uint32_t b = (uint32_t)fminf(fmaxf(x, 0.f), 4095.f);
        bin[j] = b;
      }
      if (full) {
#pragma unroll
        for (int j = 0; j < PER; ++j) atomicAdd(&sh.bins[bin[j]], 1u);
      } else {
#pragma unroll
        for (int j = 0; j < PER; ++j)
          if ((vm >> j) & 1u) atomicAdd(&sh.bins[bin[j]], 1u);
      }
      __syncthreads();
      if (wave == 0) wave_find_desc(sh.bins, kHistBins, k, &sh.s_digit, &sh.s_before);
      __syncthreads();
      const uint32_t bstar = sh.s_digit;
      const uint32_t need1 = k - sh.s_before;
      {
        uint32_t hm = 0;
#pragma unroll
        for (int j = 0; j < PER; ++j) hm |= bin[j] == bstar ? (1u << j) : 0u;
        hm &= vm;
        const uint32_t hits = __popc(hm);
        const uint32_t incl = wave_inclusive_scan(hits);
        uint32_t base = 0;
        if (lane == 63 && incl) base = atomicAdd(&sh.s_ncand, incl);
        base = __builtin_amdgcn_readlane(base, 63);
        uint32_t pos = base + incl - hits;
        while (hm) {
          const int j = __ffs((int)hm) - 1;
          hm &= hm - 1u;
          if (pos < 64u) sh.cand_sel[pos] = key[j];
          ++pos;
        }
      }
      __syncthreads();
      const uint32_t n_cand = sh.s_ncand;
      if (n_cand <= 64u) {
        // rank the candidates by their keys: the threshold is the key with fewer than need1 keys
        // above it and at least need1 at or above it
        if (wave == 0) {
          const uint32_t mine = lane < (int)n_cand ? sh.cand_sel[lane] : 0u;
          uint32_t gt = 0, ge = 0;
          for (int j = 0; j < (int)n_cand; ++j) {
            const uint32_t o = (uint32_t)__builtin_amdgcn_readlane((int)mine, j);
            gt += o > mine ? 1u : 0u;
            ge += o >= mine ? 1u : 0u;
          }
          if (lane < (int)n_cand && gt < need1 && ge >= need1) {   // every such lane holds the same key
            sh.s_T = mine;
            sh.s_need = need1 - gt;
            // entries equal to T share its bin, so all of them are candidates: ge == need1 means
            // the entries at or above T are exactly k
            sh.s_all_eq = ge == need1 ? 1u : 0u;
          }
        }
        resolved = true;
      } else {
        for (int i = tid; i < kHistBins; i += NT) sh.bins[i] = 0u;
        if (tid == 0) sh.s_ncand = 0u;
        __syncthreads();
      }
    }
  }
  if (!resolved) {
    if constexpr (RAW) {
#pragma unroll
      for (int j = 0; j < PER; ++j) key[j] = canonical_key(key[j]);
    }
    // level 1: top 12 key bits of every entry (all lanes active: one LDS atomic instruction covers 64)
#pragma unroll
    for (int j = 0; j < PER; ++j)
      if ((vm >> j) & 1u) atomicAdd(&sh.bins[key[j] >> kHistShift], 1u);
    __syncthreads();
    if (wave == 0) wave_find_desc(sh.bins, kHistBins, k, &sh.s_digit, &sh.s_before);
    __syncthreads();
    const uint32_t bstar = sh.s_digit;
    const uint32_t need1 = k - sh.s_before;   // entries still to take from bin b* (>= 1)
    // the entries of bin b* become candidates: their keys are appended to LDS with one atomic per
    // wave, a lane's after those of the lanes below it
    {
      uint32_t hm = 0;   // bit j: entry j is in b*
#pragma unroll
      for (int j = 0; j < PER; ++j) hm |= (((vm >> j) & 1u) && (key[j] >> kHistShift) == bstar) ? (1u << j) : 0u;
      const uint32_t hits = __popc(hm);
      const uint32_t incl = wave_inclusive_scan(hits);
      uint32_t base = 0;
      if (lane == 63 && incl) base = atomicAdd(&sh.s_ncand, incl);
      base = __builtin_amdgcn_readlane(base, 63);
      uint32_t pos = base + incl - hits;
      while (hm) {
        const int j = __ffs((int)hm) - 1;
        hm &= hm - 1u;
        if (pos < (uint32_t)kCandMax) sh.cand_sel[pos] = key[j];
        ++pos;
      }
    }
    __syncthreads();
    const uint32_t n_cand = sh.s_ncand;
    if (n_cand <= (uint32_t)kCandMax) {
      // wave 0 alone resolves the 20 low key bits among the candidates (two 10-bit levels in a
      // wave-private histogram); LDS operations of one wave complete in order
      if (wave == 0) {
        uint32_t prefix = bstar, need = need1;
#pragma unroll 1
        for (int lvl = 0; lvl < 2; ++lvl) {
          const int shift = kHistShift - 10 * (lvl + 1);   // 10, then 0
#pragma unroll
          for (int i = 0; i < 1024; i += 256) *(uint4*)&sh.bins[i + 4 * lane] = make_uint4(0u, 0u, 0u, 0u);
          __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
          __builtin_amdgcn_wave_barrier();
          // four candidates per lane per pass: their reads are all in flight before the first atomic
          for (uint32_t i0 = 0; i0 < n_cand; i0 += 256) {
            uint32_t kk[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const uint32_t i = i0 + 64 * u + lane;
              kk[u] = sh.cand_sel[i < n_cand ? i : 0];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const uint32_t i = i0 + 64 * u + lane;
              if (i < n_cand && (kk[u] >> (shift + 10)) == prefix) atomicAdd(&sh.bins[(kk[u] >> shift) & 1023u], 1u);
            }
          }
          __builtin_amdgcn_s_waitcnt(0xc07f);
          __builtin_amdgcn_wave_barrier();
          wave_find_desc(sh.bins, 1024, need, &sh.s_digit, &sh.s_before);
          __builtin_amdgcn_s_waitcnt(0xc07f);
          __builtin_amdgcn_wave_barrier();
          prefix = (prefix << 10) | sh.s_digit;
          need -= sh.s_before;
        }
        if (lane == 0) {
          sh.s_T = prefix;
          sh.s_need = need;
          sh.s_all_eq = 0u;
        }
      }
    } else {
      // many entries share b* (heavily tied scores): levels 2 and 3 over the whole block, ten more
      // key bits each, counting only entries with the current prefix
      uint32_t prefix = bstar, need = need1;
#pragma unroll 1
      for (int lvl = 0; lvl < 2; ++lvl) {
        const int shift = kHistShift - 10 * (lvl + 1);   // 10, then 0
        for (int i = tid; i < 1024; i += NT) sh.bins[i] = 0u;
        __syncthreads();
#pragma unroll
        for (int j = 0; j < PER; ++j) {
          const bool hit = ((vm >> j) & 1u) && (key[j] >> (shift + 10)) == prefix;
          if (__any(hit) && hit) atomicAdd(&sh.bins[(key[j] >> shift) & 1023u], 1u);
        }
        __syncthreads();
        if (wave == 0) wave_find_desc(sh.bins, 1024, need, &sh.s_digit, &sh.s_before);
        __syncthreads();
        prefix = (prefix << 10) | sh.s_digit;
        need -= sh.s_before;
      }
      if (tid == 0) {
        sh.s_T = prefix;
        sh.s_need = need;
        sh.s_all_eq = 0u;
      }
    }
  }
  __syncthreads();
}

// The selected entries' indices in ascending order into sh.cand_sel[0, k): every real entry above
// T and the first `need` equal to T (index order), placed by one block scan of the per-thread
// (greater, equal) counts packed in one word (both totals stay below 2^16); when block_threshold
// found that every entry equal to T is taken (sh.s_all_eq), of the counts of entries at or above T.  idx_of(j) is the index
// of this thread's entry j; thread t's entries precede thread t+1's in index order.  Ends with a
// barrier.
template <int NT, int PER, class IdxOf>
__device__ void block_emit(const uint32_t* key, uint32_t vm, uint32_t T, uint32_t need, uint32_t k, IdxOf idx_of,
                           SelShared<NT>& sh) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  uint32_t tm, pos;   // bit j: entry j is taken; the output position of this thread's first one
  if (sh.s_all_eq) {  // block-uniform: the taken entries are those at or above T, one compare each
    uint32_t ge = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) ge |= key[j] >= T ? (1u << j) : 0u;
    tm = ge & vm;
    const uint32_t mine = __popc(tm);
    const uint32_t incl = wave_inclusive_scan(mine);
    if (lane == 63) sh.scan[wave] = incl;
    __syncthreads();
    pos = incl - mine;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) pos += w < wave ? sh.scan[w] : 0u;
  } else {
    uint32_t gm = 0, em = 0;       // bit j: entry j is above T / equal to T
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      gm |= key[j] > T ? (1u << j) : 0u;
      em |= key[j] == T ? (1u << j) : 0u;
    }
    gm &= vm;
    em &= vm;
    const uint32_t n_gt = __popc(gm), n_eq = __popc(em);
    const uint32_t mine = (n_gt << 16) | n_eq;
    const uint32_t incl = wave_inclusive_scan(mine);
    if (lane == 63) sh.scan[wave] = incl;
    __syncthreads();
    uint32_t pre = incl - mine;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) pre += w < wave ? sh.scan[w] : 0u;
    const uint32_t eq_before = pre & 0xFFFFu;
    pos = (pre >> 16) + (eq_before < need ? eq_before : need);
    const uint32_t take_eq = eq_before < need ? (need - eq_before < n_eq ? need - eq_before : n_eq) : 0u;
    // the taken entries: all above T, and the lowest-index take_eq of those equal to T
    tm = gm;
    for (uint32_t t = 0; t < take_eq; ++t) {
      const uint32_t low = em & (0u - em);
      tm |= low;
      em ^= low;
    }
  }
  int32_t* sel = (int32_t*)sh.cand_sel;
  while (tm) {
    const int j = __ffs((int)tm) - 1;
    tm &= tm - 1u;
    if (pos < k) sel[pos] = idx_of(j);
    ++pos;
  }
  __syncthreads();
}


// Exact selection over a whole score row by one block: three radix levels (12, 10, 10 bits of the
// order key) over the row, then one pass in index order that places the selected entries with
// block scans.  Reads the row four times; the fallback of the sketch path.
template <int NT>
__device__ void select_streamed(const TopkArgs& a, int q, int64_t nv, uint32_t k, SelShared<NT>& sh,
                                int32_t* out, int32_t* rows_out, const int32_t* pt) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const float* row = a.logits + (int64_t)q * a.ld;
  uint32_t prefix = 0u, need = k;
  int pbits = 0;
#pragma unroll 1
  for (int lvl = 0; lvl < 3; ++lvl) {
    const int wdt = lvl == 0 ? 12 : 10;
    const int nb = 1 << wdt;
    const int shift = 32 - pbits - wdt;
    for (int i = tid; i < nb; i += NT) sh.bins[i] = 0u;
    __syncthreads();
    for (int64_t c = (int64_t)tid * 4; c < nv; c += (int64_t)NT * 4) {
      // rows are 16-byte aligned and ld is a multiple of 64, so the 4-entry load stays in the row
      const float4 x = *(const float4*)(row + c);
      const float v[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t key = order_key(v[e]);
        if (c + e < nv && (pbits == 0 || (key >> (32 - pbits)) == prefix))
          atomicAdd(&sh.bins[(key >> shift) & (uint32_t)(nb - 1)], 1u);
      }
    }
    __syncthreads();
    if (wave == 0) wave_find_desc(sh.bins, nb, need, &sh.s_digit, &sh.s_before);
    __syncthreads();
    prefix = (prefix << wdt) | sh.s_digit;
    pbits += wdt;
    need -= sh.s_before;
    __syncthreads();
  }
  const uint32_t T = prefix;
  // placement in index order, 4 consecutive entries per thread and NT * 4 per pass
  uint32_t gt_run = 0u, eq_run = 0u;   // selected-above / equal counts of earlier passes
  for (int64_t base = 0; base < nv; base += (int64_t)NT * 4) {
    const int64_t c0 = base + (int64_t)tid * 4;
    uint32_t gm = 0u, em = 0u;
    if (c0 < nv) {
      const float4 x = *(const float4*)(row + c0);
      const float v[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t key = order_key(v[e]);
        const bool ok = c0 + e < nv;
        gm |= (ok && key > T) ? (1u << e) : 0u;
        em |= (ok && key == T) ? (1u << e) : 0u;
      }
    }
    const uint32_t n_gt = __popc(gm), n_eq = __popc(em);
    const uint32_t mine = (n_gt << 16) | n_eq;
    const uint32_t incl = wave_inclusive_scan(mine);
    if (lane == 63) sh.scan[wave] = incl;
    __syncthreads();
    uint32_t pre = incl - mine, tot = 0u;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
      pre += w < wave ? sh.scan[w] : 0u;
      tot += sh.scan[w];
    }
    __syncthreads();   // sh.scan is rewritten by the next pass
    const uint32_t eq_before = eq_run + (pre & 0xFFFFu);
    uint32_t pos = gt_run + (pre >> 16) + (eq_before < need ? eq_before : need);
    uint32_t take_eq = eq_before < need ? (need - eq_before < n_eq ? need - eq_before : n_eq) : 0u;
    uint32_t tm = gm;
    for (uint32_t t = 0; t < take_eq; ++t) {
      const uint32_t low = em & (0u - em);
      tm |= low;
      em ^= low;
    }
    while (tm) {
      const int e = __ffs((int)tm) - 1;
      tm &= tm - 1u;
      if (pos < k) {
        const int c = (int)(c0 + e);
        out[pos] = c;
        if (rows_out) {
          const int pg = pt[c >> 6];
          rows_out[pos] = (unsigned)pg < (unsigned)a.num_pages ? pg * kPage + (c & (kPage - 1)) : -1;
        }
      }
      ++pos;
    }
    gt_run += tot >> 16;
    eq_run += tot & 0xFFFFu;
    if (gt_run + (eq_run < need ? eq_run : need) >= k) break;   // block-uniform
  }
}

}  // namespace csa
