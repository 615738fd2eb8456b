// C4 indexer page scores on gfx950: the device code shared by the indexer kernels and the
// long-row selection, which rescores a row when its sketches cannot decide it.
//
// Score of compressed entry c for one query ([P1] "DeepSeek-V4 全面解读" section 2.10, forward steps
// 5-8; [P2] "DeepSeek-V4 in SGLang 深度理解分析" concept 3 / algorithm 2):
//     s[c] = sum_h w[h] * max(0, qI[h] . kI[c])
// with FP8 E4M3FN or FP4 E2M1 operands that carry one E8M0 scale per 32 elements.
//
// FP8 path: the scores go through the bf16 matrix cores (v_mfma_f32_16x16x32_bf16), not the
// FP8 ones.  Measured on gfx950, the FP8 instructions (v_mfma_f32_16x16x32_fp8_fp8 and the scaled
// v_mfma_scale_f32_16x16x128_f8f6f4) sum each run of eight products on a fixed-point grid about
// 16 bits below the largest of them: 448*448 + 1.75 comes back as 448*448, and
// 448*448 - 448*448 + 0.125 as 0.  On random E4M3 operands the error reaches 1.4e-4 of the sum
// of |products|, and on the 8192-token causal prefill it moved scores by up to 5.8e-5, enough to
// swap the 512th and 513th entries of rows whose cut falls near a score of zero.  The bf16
// instruction keeps every product exact and rounds like fp32 (2.6e-7 of the sum of |products|
// on the same operands).  Every E4M3 value times a power-of-two scale is a bf16 value, so
// v_cvt_scalef32_pk_bf16_fp8 converts two codes per instruction exactly, folding the E8M0 block
// scale in (scale bytes 10..245 keep every converted value a normal bf16).  Operand layout: lane
// l = n + 16*g holds bytes [16g, 16g+16) and [64+16g, 64+16g+16) of row n (the query head, or
// the key 4n+kg of key group kg), i.e. elements of scale blocks g/2 and 2 + g/2; the four
// 16x16x32 MFMAs of a key group take the lane's bytes eight at a time, and A and B use the same
// layout, so codes pair up element by element.  A wave scores one page (64 entries) per step:
// MFMA column n of key group kg is slot 4n+kg.  The epilogue applies ReLU and the head weights,
// then a 2-step reduce-scatter over the four lane groups leaves lane l with the full score of
// slot 4*(l%16) + l/16.  Decode: keys stream straight from HBM into VGPRs (no LDS), each lane
// loads 2 x 16 B per key group, and each page is read exactly once.  Causal prefill, where all
// queries share one request's keys, stages key pages in LDS per block of queries instead (see
// below).
//
// FP4 path (two E2M1 codes per byte, element 2i in the low nibble): the scaled instruction
// v_mfma_scale_f32_16x16x128_f8f6f4 with both operand formats set to FP4, which reads four
// registers per lane.  Lane l = m + 16*g's 32 codes all fall in scale block g (measured on gfx950),
// so lane (m, g) loads the one contiguous 16-byte chunk of row m that holds elements [32g, 32g+32)
// and its scale operands are the stored block scales.  E2M1 products are multiples of 1/4 below
// 36, so every run of them is exact on the instruction's grid (measured: no error on random
// operands).  Rows are 64 bytes, a key page 4 KB: half the FP8 key traffic.
#pragma once

#include "csa_device.h"
#include "csa_internal.h"

namespace csa {

// bytes of one 128-dim operand row
template <bool FP4>
constexpr int kRowB = FP4 ? kDI / 2 : kDI;

template <int HG, int KG>
__device__ __forceinline__ v4f mma_fp4(const v8i& a, const v8i& b, int sa, int sb, v4f c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 4, HG, sa, KG, sb);
}

__device__ __forceinline__ v4f mma_bf16x32(const v8bf& a, const v8bf& b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// E8M0 scale byte e -> 2^(e - 127) (bytes 1..254)
__device__ __forceinline__ float e8m0_float(uint32_t e) { return __uint_as_float(e << 23); }

// eight E4M3FN codes (two dwords) times the power of two s, as bf16 (exact)
__device__ __forceinline__ v8bf fp8x8_bf16(uint32_t w0, uint32_t w1, float s) {
  const v2bf a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, s, false);
  const v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, s, true);
  const v2bf c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, s, false);
  const v2bf d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, s, true);
  return v8bf{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// A lane's FP8 operand (bytes [16g, +16) scaled by s_lo, bytes [64+16g, +16) by s_hi) as the
// B/A operands of four 16x16x32 bf16 MFMAs
__device__ __forceinline__ void fp8_operand_bf16(const v8i& r, float s_lo, float s_hi, v8bf* o) {
  o[0] = fp8x8_bf16((uint32_t)r[0], (uint32_t)r[1], s_lo);
  o[1] = fp8x8_bf16((uint32_t)r[2], (uint32_t)r[3], s_lo);
  o[2] = fp8x8_bf16((uint32_t)r[4], (uint32_t)r[5], s_hi);
  o[3] = fp8x8_bf16((uint32_t)r[6], (uint32_t)r[7], s_hi);
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
template <bool FP4, bool NT = true>
__device__ __forceinline__ v8i load_key_operand(const uint8_t* lane_base, int kg) {
  constexpr int halves = FP4 ? 1 : 2;
  const v4u lo = load16<NT>(lane_base + kg * halves * 1024);
  v8i r;
  r[0] = (int)lo[0]; r[1] = (int)lo[1]; r[2] = (int)lo[2]; r[3] = (int)lo[3];
  if constexpr (FP4) {
    r[4] = 0; r[5] = 0; r[6] = 0; r[7] = 0;
  } else {
    const v4u hi = load16<NT>(lane_base + (kg * halves + 1) * 1024);
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


// One query's indexer heads as MFMA A operands (padded heads zeroed) and the head weights of this
// lane's output rows.  FP4: the codes and their E8M0 block scales, one byte per head group.  FP8:
// converted to bf16 once, with the lane's two block scales folded in.
template <int NHG, bool FP4>
struct QueryOps {
  v8i raw[FP4 ? NHG : 1];
  v8bf bf[FP4 ? 1 : NHG][4];
  int qsc;
  float wv[NHG][4];
};

// The loads of an FP8 query (codes, the lane's two block scales, head weights), apart from the
// conversion, so that the causal prefill can have the next query's loads in flight while it
// scores the current one.
template <int NHG>
struct QueryRawFp8 {
  v8i raw[NHG];
  uint32_t sc[NHG];     // scale bytes of blocks g/2 (bits 0-7) and 2 + g/2 (bits 8-15)
  float wv[NHG][4];
};

template <int NHG>
__device__ __forceinline__ void fetch_query_fp8(const IndexerArgs& a, int q, int n, int g, QueryRawFp8<NHG>& R) {
  const uint8_t* qb = (const uint8_t*)a.qI + (int64_t)q * a.HI * kDI;
#pragma unroll
  for (int hg = 0; hg < NHG; ++hg) {
    const int h = 16 * hg + n;
    const int hc = h < a.HI ? h : a.HI - 1;
    const v8i v = load_row_operand<false>(qb + hc * kDI, g);
    const uint8_t* sp = a.qI_scale + ((int64_t)q * a.HI + hc) * 4;
    const bool ok = h < a.HI;
#pragma unroll
    for (int e = 0; e < 8; ++e) R.raw[hg][e] = ok ? v[e] : 0;
    R.sc[hg] = (uint32_t)sp[g >> 1] | ((uint32_t)sp[2 + (g >> 1)] << 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hh = 16 * hg + 4 * g + i;
      const float x = a.w[(int64_t)q * a.HI + (hh < a.HI ? hh : a.HI - 1)];
      R.wv[hg][i] = hh < a.HI ? x : 0.f;
    }
  }
}

template <int NHG>
__device__ __forceinline__ void set_query_fp8(const QueryRawFp8<NHG>& R, QueryOps<NHG, false>& Q) {
#pragma unroll
  for (int hg = 0; hg < NHG; ++hg) {
    const float s_lo = e8m0_float(R.sc[hg] & 0xFFu), s_hi = e8m0_float((R.sc[hg] >> 8) & 0xFFu);
    fp8_operand_bf16(R.raw[hg], s_lo, s_hi, Q.bf[hg]);
#pragma unroll
    for (int i = 0; i < 4; ++i) Q.wv[hg][i] = R.wv[hg][i];
  }
}

template <int NHG, bool FP4>
__device__ __forceinline__ void load_query(const IndexerArgs& a, int q, int n, int g, QueryOps<NHG, FP4>& Q) {
  if constexpr (FP4) {
    const uint8_t* qb = (const uint8_t*)a.qI + (int64_t)q * a.HI * kRowB<true>;
    Q.qsc = 0;
#pragma unroll
    for (int hg = 0; hg < NHG; ++hg) {
      const int h = 16 * hg + n;
      const int hc = h < a.HI ? h : a.HI - 1;
      const v8i v = load_row_operand<true>(qb + hc * kRowB<true>, g);
      const bool ok = h < a.HI;
#pragma unroll
      for (int e = 0; e < 8; ++e) Q.raw[hg][e] = ok ? v[e] : 0;
      Q.qsc |= (ok ? (int)a.qI_scale[((int64_t)q * a.HI + hc) * 4 + g] : 127) << (8 * hg);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int hh = 16 * hg + 4 * g + i;
        const float x = a.w[(int64_t)q * a.HI + (hh < a.HI ? hh : a.HI - 1)];
        Q.wv[hg][i] = hh < a.HI ? x : 0.f;
      }
    }
  } else {
    QueryRawFp8<NHG> R;
    fetch_query_fp8<NHG>(a, q, n, g, R);
    set_query_fp8(R, Q);
  }
}

// Score of one page (64 entries) for one query: 4 x NHG MFMAs (FP4: scaled 16x16x128; FP8: four
// 16x16x32 bf16 per key group and head group), ReLU and head weights, then a reduce-scatter over the four lane groups leaves lane (n, g) with the score of slot 4n + g.
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

// One key group of a page against one query (bf16 operands): NHG x 4 MFMAs, then ReLU and the
// head weights summed over this lane's four output rows of every head group.
template <int NHG, class QOp>
__device__ __forceinline__ float key_group_bf16(QOp qop, const float (*wv)[4], const v8bf* kf) {
  v4f acc[NHG];
#pragma unroll
  for (int hg = 0; hg < NHG; ++hg) acc[hg] = v4f{0.f, 0.f, 0.f, 0.f};
  // j outer, heads inner: consecutive MFMAs are independent
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int hg = 0; hg < NHG; ++hg) acc[hg] = mma_bf16x32(qop(hg, j), kf[j], acc[hg]);
  float sacc = 0.f;
#pragma unroll
  for (int hg = 0; hg < NHG; ++hg)
#pragma unroll
    for (int e = 0; e < 4; ++e) sacc = fmaf(wv[hg][e], relu(acc[hg][e]), sacc);
  return sacc;
}

// lanes 0-31 keep key groups 0 and 1, lanes 32-63 key groups 2 and 3; then even rows keep the
// first of the pair and odd rows the second: lane (n, g) ends with the score of slot 4n + g
__device__ __forceinline__ float reduce_key_groups(const float* part) {
  const float k0 = swap_sum32(part[0], part[2]);
  const float k1 = swap_sum32(part[1], part[3]);
  return swap_sum16(k0, k1);
}

// ks_lo / ks_hi: the page's scale words this lane needs.  FP4: word l of the page's [4 blocks]
// [64 slots] scale array (block g of slots 4n..4n+3; the key group picks the byte).  FP8: words
// 16*(g/2) + n and 16*(2 + g/2) + n (blocks g/2 and 2 + g/2 of the same slots).
template <int NHG, bool FP4>
__device__ __forceinline__ float score_page(const QueryOps<NHG, FP4>& Q, const v8i* kb, uint32_t ks_lo,
                                            uint32_t ks_hi) {
  float part[4];
  if constexpr (FP4) {
    v4f acc[NHG][4];
    static_for<0, NHG>::run([&](auto HGc) {
      constexpr int HG = decltype(HGc)::value;
      static_for<0, 4>::run([&](auto KGc) {
        constexpr int KG = decltype(KGc)::value;
        acc[HG][KG] = mma_fp4<HG, KG>(Q.raw[HG], kb[KG], Q.qsc, (int)ks_lo, v4f{0.f, 0.f, 0.f, 0.f});
      });
    });
#pragma unroll
    for (int kg = 0; kg < 4; ++kg) {
      float sacc = 0.f;
#pragma unroll
      for (int hg = 0; hg < NHG; ++hg)
#pragma unroll
        for (int e = 0; e < 4; ++e) sacc = fmaf(Q.wv[hg][e], relu(acc[hg][kg][e]), sacc);
      part[kg] = sacc;
    }
  } else {
    auto qop = [&](int hg, int j) -> const v8bf& { return Q.bf[hg][j]; };
#pragma unroll
    for (int kg = 0; kg < 4; ++kg) {
      v8bf kf[4];
      fp8_operand_bf16(kb[kg], e8m0_float((ks_lo >> (8 * kg)) & 0xFFu), e8m0_float((ks_hi >> (8 * kg)) & 0xFFu), kf);
      part[kg] = key_group_bf16<NHG>(qop, Q.wv, kf);
    }
  }
  return reduce_key_groups(part);
}

// The scale words of one key page that lane (n, g) needs (see score_page)
template <bool FP4>
__device__ __forceinline__ void page_scale_words(const uint8_t* page_scales, int n, int g, uint32_t& lo, uint32_t& hi) {
  const uint32_t* w = (const uint32_t*)page_scales;
  if constexpr (FP4) {
    lo = w[n + 16 * g];
    hi = 0u;
  } else {
    lo = w[n + 16 * (g >> 1)];
    hi = w[n + 16 * (2 + (g >> 1))];
  }
}

// Rescoring of one span of kSketchSpan entries (the eight pages one decode-kernel wave scores) of
// query q's row into a.logits, for the visible entries of the span.  The long-row decode does not
// store its scores (its selection works from the per-wave sketches); when the sketches cannot
// decide a row's top k, the selection rescores the row with this.  Same operands, the same matrix-
// core chains and the same fp32 sums in the same order as score_page, so the same scores; but a
// page, a head group and a key group at a time (query and key operands reloaded through the caches
// as needed), which fits in far fewer registers than the decode kernel's resident operands.
template <int NHG, bool FP4>
__device__ __forceinline__ void rescore_span(const IndexerArgs& a, int q, int64_t span, int lane) {
  constexpr int kSpanPages = kSketchSpan / kPage;
  const int n = lane & 15, g = lane >> 4;
  int r;
  const int64_t nv = visible_count(a, q, r);
  const int64_t p_first = span * kSpanPages;
  if (p_first * kPage >= nv) return;
  const int32_t* pt = a.page_table + (int64_t)(r < 0 ? 0 : r) * a.max_pages;
  const uint8_t* keys = (const uint8_t*)a.keys;
  const int64_t vis_pages = (nv + kPage - 1) / kPage;
  int my_pid = -1;
  if (lane < kSpanPages && p_first + lane < vis_pages) my_pid = pt[p_first + lane];
  const uint8_t* qrow = (const uint8_t*)a.qI + (int64_t)q * a.HI * kRowB<FP4>;
  float* lrow = a.logits + (int64_t)q * a.ld;
#pragma unroll 1
  for (int i = 0; i < kSpanPages; ++i) {
    const int pid_raw = __builtin_amdgcn_readlane(my_pid, i);
    const bool mapped = (unsigned)pid_raw < (unsigned)a.num_pages;
    const int pid = mapped ? pid_raw : 0;
    const uint8_t* kp = keys + (int64_t)pid * (kPage * kRowB<FP4>) + 16 * lane;
    uint32_t ks_lo, ks_hi;
    page_scale_words<FP4>(a.kscale + (int64_t)pid * 256, n, g, ks_lo, ks_hi);
    float sacc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
    for (int hg = 0; hg < NHG; ++hg) {
      // an opaque zero keeps this head group's query loads and the key conversions inside the
      // loop, so only one head group's operands are live at a time
      int z = 0;
      asm volatile("" : "+s"(z));
      const uint32_t lo = ks_lo ^ (uint32_t)z, hi = ks_hi ^ (uint32_t)z;
      // this head group's operands, as load_query forms them
      const int h = 16 * hg + n;
      const int hc = h < a.HI ? h : a.HI - 1;
      const bool ok = h < a.HI;
      float wv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int hh = 16 * hg + 4 * g + e;
        const float x = a.w[(int64_t)q * a.HI + (hh < a.HI ? hh : a.HI - 1)];
        wv[e] = hh < a.HI ? x : 0.f;
      }
      const v8i qv = load_row_operand<FP4>(qrow + z + hc * kRowB<FP4>, g);
      v8i raw;
#pragma unroll
      for (int e = 0; e < 8; ++e) raw[e] = ok ? qv[e] : 0;
      const uint8_t* sp = a.qI_scale + ((int64_t)q * a.HI + hc) * 4;
      v8bf qb[4];
      int qsc = 127;
      if constexpr (FP4) {
        qsc = ok ? (int)sp[g] : 127;
      } else {
        fp8_operand_bf16(raw, e8m0_float(sp[g >> 1]), e8m0_float(sp[2 + (g >> 1)]), qb);
      }
      static_for<0, 4>::run([&](auto KGc) {
        constexpr int kg = decltype(KGc)::value;
        // the key group's operand bytes, reloaded (through the caches) for every head group
        const v8i kb = load_key_operand<FP4, false>(kp + z, kg);
        v4f acc;
        if constexpr (FP4) {
          acc = mma_fp4<0, kg>(raw, kb, qsc, (int)lo, v4f{0.f, 0.f, 0.f, 0.f});
        } else {
          v8bf kf[4];
          fp8_operand_bf16(kb, e8m0_float((lo >> (8 * kg)) & 0xFFu), e8m0_float((hi >> (8 * kg)) & 0xFFu), kf);
          acc = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int j = 0; j < 4; ++j) acc = mma_bf16x32(qb[j], kf[j], acc);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) sacc[kg] = fmaf(wv[e], relu(acc[e]), sacc[kg]);
      });
    }
    const float score = reduce_key_groups(sacc);
    const int64_t c = (p_first + i) * kPage + 4 * n + g;
    if (c < nv) lrow[c] = mapped ? score : -INFINITY;
  }
}
}  // namespace csa
