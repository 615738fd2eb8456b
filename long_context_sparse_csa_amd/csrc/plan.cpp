// Host-side planning of the kernel launches: which selection and attention variants a call takes
// and how much workspace they need.  Plain host code, shared by the GPU build and the host-only
// (sanitizer) build of the C ABI layer.
#include <cstdlib>

#include "csa_internal.h"

namespace csa {

// Heads per block of the matrix-core kernels: 64 (one block per query and key range, q read once
// per range, each dequantised tile serving four head groups) unless the heads fit one group of 16,
// or the batch is small and its lists short: with few queries, 16-head blocks fill the GPU with
// four times as many blocks per key range, so each range can stay longer (measured on decode with
// 64 heads and 640 slots: 8 queries take 13.8 us in 16-head blocks against 19.0 us in 64-head
// blocks; 32 queries take 22.5 against 20.8).  Long lists have key ranges enough to fill the GPU
// with 64-head blocks, and 16-head blocks would gather every row four times (8 queries of 8,320
// slots: 27.7 us in 64-head blocks, 80.1 us in 16-head blocks).
constexpr int kSmallBatchSlots = 2048;

int attn_head_block(int Q, int H, int n_idx) {
  static const int forced = [] {
    const char* e = getenv("CSA_ATTN_HEADS");   // tuning override: 16 or 64
    return e ? atoi(e) : 0;
  }();
  if (forced == 16 || forced == 64) return forced;
  return ((H + 15) / 16 == 1 || (Q <= 16 && n_idx <= kSmallBatchSlots)) ? 16 : 64;
}

int plan_attn_split(int Q, int H, int n_idx, int q_dt) {
  if (q_dt == 0) return 1;
  static const int forced = [] {
    const char* e = getenv("CSA_ATTN_SPLIT");   // tuning override: fixed split count
    return e ? atoi(e) : 0;
  }();
  const int n_tiles = (n_idx + kTile - 1) / kTile;
  // a block holds at most kMaxSlots slots (n_idx <= kMaxSplit * kMaxSlots keeps this within kMaxSplit)
  const int min_s = (n_tiles + kMaxSlots / kTile - 1) / (kMaxSlots / kTile);
  if (forced > 0) {
    const int f = forced < kMaxSplit ? (forced < n_tiles ? forced : n_tiles) : (kMaxSplit < n_tiles ? kMaxSplit : n_tiles);
    return f > min_s ? f : min_s;
  }
  const int hb = attn_head_block(Q, H, n_idx);
  const int hchunks = (((H + 15) & ~15) + hb - 1) / hb;
  const int blocks = Q * hchunks;
  int s = (256 + blocks - 1) / blocks;
  const int max_s = n_tiles / 2 > 1 ? n_tiles / 2 : 1;
  if (s > max_s) s = max_s;
  if (s > kMaxSplit) s = kMaxSplit;
  if (s < min_s) s = min_s;
  if (s < 1) s = 1;
  // as few splits as give each block the same number of tiles: 20 tiles over 8 splits are 3 tiles
  // a block and an 8th block with none, which would still select and write an empty partial that
  // the merge reads (7 splits here)
  if (n_tiles > 0) {
    const int tps = (n_tiles + s - 1) / s;
    s = (n_tiles + tps - 1) / tps;
  }
  return s;
}

size_t attn_partial_bytes(int Q, int H, int n_idx) {
  const int s = plan_attn_split(Q, H, n_idx, 1);
  if (s <= 1) return 0;
  const size_t Hpad = (size_t)((H + 15) & ~15);
  return (size_t)Q * s * Hpad * (kRowD * sizeof(uint16_t) + 4 * sizeof(float));   // fp16 rows + (m, l, amax)
}

bool attn_uses_matrix_cores(int q_dt, int win_fmt, int comp_fmt, int n_win, int n_comp) {
  if (q_dt != 1) return false;
  const bool w_ok = n_win == 0 || win_fmt == kRowBF16 || win_fmt == kRowFP8;
  const bool c_ok = n_comp == 0 || comp_fmt == kRowBF16 || comp_fmt == kRowFP8;
  return w_ok && c_ok;
}

bool topk_single_ok(int64_t max_n_vis, int k) { return max_n_vis <= kSingleMax && k <= kSingleMax; }

// Long rows of a decode take the sketches when every row of the longest
// length has at least 4 k of them (so the k-th largest lies well inside), up to 2^20 entries.
bool topk_sketch_ok(int64_t max_n_vis, int k) {
  const int64_t waves = (max_n_vis + kSketchSpan - 1) / kSketchSpan;
  return k <= kSingleMaxK && waves <= kSketchMaxWaves && waves * kSketchTop >= 4 * (int64_t)k;
}

int64_t topk_sketch_waves(int64_t max_n_vis) { return (max_n_vis + kSketchSpan - 1) / kSketchSpan; }

int64_t sketch_rescore_from(int k) { return (int64_t)((k + kSketchTop - 1) / kSketchTop) * kSketchSpan; }

}  // namespace csa
