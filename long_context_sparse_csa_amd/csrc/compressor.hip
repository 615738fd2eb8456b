// Compressor: writes compressed entries into the paged caches the path reads ([P1] "DeepSeek-V4
// 全面解读" section 2.9, Compressor; section 2.6 apply_rotary_emb; section 2.7 rotate_activation;
// [P2] "DeepSeek-V4 in SGLang 深度理解分析" concept 2).
//
// Entry c pools a window of `ratio` tokens.  At ratio 4 the windows overlap: every token carries
// two projection halves of D features, the overlapping half [0, D) lent to the next window and
// the normal half [D, 2D) used by its own, so entry c pools the previous window's overlapping
// halves and its own normal halves (2 x 4 positions; entry 0 has no previous window).  At ratio
// 128 it pools its 128 tokens.  Per feature: gate score + position embedding, softmax over the
// positions, weighted sum of the kv projections; then RMSNorm over the row, rotary embedding of
// the last 64 features as consecutive (re, im) pairs, and for the indexer's keys a Hadamard
// rotation of the whole row.  The row is quantised into the cache format and written to page
// page_table[c >> 6], slot c & 63.
//
// A thread owns 8 consecutive features (4 rotary pairs): one 16-byte load of bf16 projections
// (two of fp32) per window position, so a token row is read by D/8 lanes with no redundancy and
// all positions' loads are issued before the softmax needs them.  A 512-feature entry is one wave
// (four entries per block), a 128-feature key 16 lanes (sixteen keys per block); the row-wide
// reductions (RMSNorm, block maxima) and the Hadamard stages across lanes are lane exchanges.  The
// kernel is HBM-bound: it reads coff * D * 2 projections per token once and writes one cache row
// per entry.
#include "csa_device.h"
#include "csa_internal.h"

namespace csa {

// 8 projections of a row: bf16 (one 16-byte load) or fp32 (two)
template <bool BF16>
__device__ __forceinline__ void load8(const void* base, int64_t off, float* v) {
  if constexpr (BF16) {
    const uint4 w = *(const uint4*)((const uint16_t*)base + off);
    const uint32_t x[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_bits_to_f32(x[i] & 0xFFFFu);
      v[2 * i + 1] = bf16_bits_to_f32(x[i] >> 16);
    }
  } else {
    const float4 a = *(const float4*)((const float*)base + off);
    const float4 b = *(const float4*)((const float*)base + off + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

// nearest E2M1 code of |x| <= 6 (larger saturates), ties to the even code; sign in bit 3
__device__ __forceinline__ uint32_t e2m1_code(float x) {
  const float a = fabsf(x);
  uint32_t c;
  if (a <= 0.25f) c = 0;
  else if (a < 0.75f) c = 1;
  else if (a <= 1.25f) c = 2;
  else if (a < 1.75f) c = 3;
  else if (a <= 2.5f) c = 4;
  else if (a < 3.5f) c = 5;
  else if (a <= 5.0f) c = 6;
  else c = 7;
  return (x < 0.f && c != 0) ? (c | 8u) : c;
}

// biased E8M0 exponent of the power-of-two scale 2^ceil(log2(v)) for a normal positive v: the
// exponent field, plus one when any mantissa bit is set
__device__ __forceinline__ uint32_t e8m0_ceil(float v) {
  const uint32_t b = __float_as_uint(v);
  const uint32_t e = ((b >> 23) & 0xFFu) + ((b & 0x7FFFFFu) != 0u ? 1u : 0u);
  return e > 254u ? 254u : e;
}

// max / sum over the L lanes of an aligned lane group
template <int L>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int m = 1; m < L; m <<= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}
template <int L>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int m = 1; m < L; m <<= 1) v += __shfl_xor(v, m);
  return v;
}

// BF16 is a template parameter so that every position's loads are straight-line code the compiler
// can issue together (a run-time format test put a branch around each load)
// Byte offset of byte b of key row r (0..63) of index-key page pid in the operand-order page the
// indexer reads (FP8: 128-byte rows, FP4: 64-byte rows): row r = 4n + kg and bytes
// [64h + 16g, +16) form the 16-byte chunk of lane n + 16g in kilobyte kg·halves + h.
template <bool FP4>
__device__ __forceinline__ int64_t key_byte(int pid, int r, int b) {
  constexpr int halves = FP4 ? 1 : 2;
  const int kg = r & 3, n = r >> 2, h = b >> 6, g = (b >> 4) & 3;
  return (int64_t)pid * (kPage * 64 * halves) + (kg * halves + h) * 1024 + (n + 16 * g) * 16 + (b & 15);
}

template <int D, bool BF16>
__global__ __launch_bounds__(256) void compress_kernel(CompressArgs a) {
  constexpr int L = D / 8;                 // lanes per entry
  constexpr int kRope = 64;
  const int lane_in = threadIdx.x % L;     // features [8 lane_in, 8 lane_in + 8)
  const int64_t ci = (int64_t)blockIdx.x * (256 / L) + threadIdx.x / L;   // entry index in the call
  if (ci >= a.c_count) return;             // whole lane groups leave together
  const int64_t c = a.c_begin + ci;
  const bool overlap = a.ratio == 4;
  const int coff = overlap ? 2 : 1;
  const int f0 = 8 * lane_in;

  // online softmax over the window positions, per feature
  float m[8], l[8], acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    m[e] = -INFINITY;
    l[e] = 0.f;
    acc[e] = 0.f;
  }
  auto add = [&](int64_t tok, int half, int wpos) {
    const int col = half * D + f0;
    const int64_t off = (tok - a.tok0) * a.ld + col;
    float k[8], sc[8];
    load8<BF16>(a.kv, off, k);
    load8<BF16>(a.score, off, sc);
    const float4 p0 = *(const float4*)(a.ape + (int64_t)wpos * coff * D + col);
    const float4 p1 = *(const float4*)(a.ape + (int64_t)wpos * coff * D + col + 4);
    const float pe[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float s = sc[e] + pe[e];
      const float n = fmaxf(m[e], s);
      const float r = exp2f((m[e] - n) * kLog2e), x = exp2f((s - n) * kLog2e);
      l[e] = fmaf(l[e], r, x);
      acc[e] = fmaf(acc[e], r, x * k[e]);
      m[e] = n;
    }
  };
  if (overlap) {
    if (c > 0) {
#pragma unroll
      for (int w = 0; w < 4; ++w) add((c - 1) * 4 + w, 0, w);
    }
#pragma unroll
    for (int w = 0; w < 4; ++w) add(c * 4 + w, 1, w);
  } else {
#pragma unroll 4
    for (int w = 0; w < a.ratio; ++w) add(c * a.ratio + w, 0, w);
  }
  float y[8];
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    y[e] = acc[e] / l[e];
    ss = fmaf(y[e], y[e], ss);
  }

  // RMSNorm over the D features
  ss = group_sum<L>(ss);
  const float inv = 1.f / sqrtf(ss / (float)D + a.eps);
  {
    const float4 w0 = *(const float4*)(a.norm_w + f0), w1 = *(const float4*)(a.norm_w + f0 + 4);
    const float w[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = y[e] * inv * w[e];
  }

  // rotary embedding of the last 64 features: pairs (2j, 2j+1) times cos + i sin
  if (f0 >= D - kRope) {
    const int p0 = (f0 - (D - kRope)) / 2;
    const float4 cs = *(const float4*)(a.rope_cos + ci * (kRope / 2) + p0);
    const float4 sn = *(const float4*)(a.rope_sin + ci * (kRope / 2) + p0);
    const float cv[4] = {cs.x, cs.y, cs.z, cs.w}, sv[4] = {sn.x, sn.y, sn.z, sn.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float re = y[2 * j], im = y[2 * j + 1];
      y[2 * j] = re * cv[j] - im * sv[j];
      y[2 * j + 1] = re * sv[j] + im * cv[j];
    }
  }

  const int pid = a.page_table[c >> 6];
  const bool mapped = (unsigned)pid < (unsigned)a.num_pages;

  if constexpr (D == 512) {
    uint8_t* row = a.out + ((int64_t)pid * kPage + (c & (kPage - 1))) * row_bytes(a.out_fmt);
    if (a.out_fmt == kRowF32) {
      if (mapped) {
        *(float4*)(row + 4 * f0) = make_float4(y[0], y[1], y[2], y[3]);
        *(float4*)(row + 4 * f0 + 16) = make_float4(y[4], y[5], y[6], y[7]);
      }
    } else if (a.out_fmt == kRowBF16) {
      if (mapped)
        *(uint4*)(row + 2 * f0) = make_uint4(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]),
                                             pack_bf16x2(y[4], y[5]), pack_bf16x2(y[6], y[7]));
    } else {
      // e4m3fn nope with one fp32 scale per 64 features (8 lanes); every lane joins the exchange
      float amax = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(y[e]));
      amax = group_max<8>(amax);
      if (f0 < kNope) {
        const float sc = fmaxf(amax, 1e-4f) * (1.f / 448.f);
        uint32_t w[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          int v = __builtin_amdgcn_cvt_pk_fp8_f32(y[4 * h] / sc, y[4 * h + 1] / sc, 0, false);
          v = __builtin_amdgcn_cvt_pk_fp8_f32(y[4 * h + 2] / sc, y[4 * h + 3] / sc, v, true);
          w[h] = (uint32_t)v;
        }
        if (mapped) {
          *(uint2*)(row + f0) = make_uint2(w[0], w[1]);
          if ((lane_in & 7) == 0) *(float*)(row + 576 + 4 * (f0 >> 6)) = sc;
        }
      } else if (mapped) {
        *(uint4*)(row + 448 + 2 * (f0 - kNope)) = make_uint4(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]),
                                                             pack_bf16x2(y[4], y[5]), pack_bf16x2(y[6], y[7]));
        if (lane_in == L - 1) *(uint32_t*)(row + 604) = 0u;
      }
    }
  } else {
    // indexer key: Hadamard rotation over the 128 features (the butterfly of stride h pairs
    // feature e with e ^ h: inside the thread for h < 8, else lane lane_in ^ (h / 8)), then E8M0
    // per 32 features (4 lanes) and FP8 or FP4 codes
#pragma unroll
    for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if ((e & h) == 0) {
          const float u = y[e] + y[e + h], v = y[e] - y[e + h];
          y[e] = u;
          y[e + h] = v;
        }
      }
    }
#pragma unroll
    for (int h = 8; h < D; h <<= 1) {
      const bool hi = (lane_in & (h >> 3)) != 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float o = __shfl_xor(y[e], h >> 3);
        y[e] = hi ? o - y[e] : y[e] + o;
      }
    }
    const float hs = 0.08838834764831845f;   // 128^-1/2
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      y[e] *= hs;
      amax = fmaxf(amax, fabsf(y[e]));
    }
    amax = group_max<4>(amax);
    const bool fp4 = a.out_fmt == 3;
    const uint32_t ex = fp4 ? e8m0_ceil(fmaxf(amax, 6.f * 1.17549435e-38f) / 6.f)
                            : e8m0_ceil(fmaxf(amax, 1e-4f) * (1.f / 448.f));
    const float q = __uint_as_float((254u - ex) << 23);   // 2^-(ex-127), exact
    if (mapped) {
      if (fp4) {
        uint32_t w = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) w |= e2m1_code(y[e] * q) << (4 * e);
        *(uint32_t*)(a.out + key_byte<true>(pid, c & (kPage - 1), f0 / 2)) = w;
      } else {
        uint32_t w[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          int v = __builtin_amdgcn_cvt_pk_fp8_f32(y[4 * h] * q, y[4 * h + 1] * q, 0, false);
          v = __builtin_amdgcn_cvt_pk_fp8_f32(y[4 * h + 2] * q, y[4 * h + 3] * q, v, true);
          w[h] = (uint32_t)v;
        }
        *(uint2*)(a.out + key_byte<false>(pid, c & (kPage - 1), f0)) = make_uint2(w[0], w[1]);
      }
      if ((lane_in & 3) == 0) a.out_scales[(int64_t)pid * 256 + (f0 >> 5) * kPage + (c & (kPage - 1))] = (uint8_t)ex;
    }
  }
}

hipError_t launch_compress(const CompressArgs& a, hipStream_t s) {
  if (a.c_count <= 0) return hipSuccess;
  ProfScope p(a.D == 512 ? "compress_kv" : "compress_keys", s);
  const int per_block = 256 / (a.D / 8);   // entries per block of 256 threads
  const unsigned blocks = (unsigned)((a.c_count + per_block - 1) / per_block);
  const bool bf16 = a.proj_dt == 1;
  if (a.D == 512) {
    if (bf16) CSA_LAUNCH(p, (compress_kernel<512, true>), dim3(blocks), dim3(256), s, a);
    else CSA_LAUNCH(p, (compress_kernel<512, false>), dim3(blocks), dim3(256), s, a);
  } else {
    if (bf16) CSA_LAUNCH(p, (compress_kernel<128, true>), dim3(blocks), dim3(256), s, a);
    else CSA_LAUNCH(p, (compress_kernel<128, false>), dim3(blocks), dim3(256), s, a);
  }
  return hipGetLastError();
}

}  // namespace csa
