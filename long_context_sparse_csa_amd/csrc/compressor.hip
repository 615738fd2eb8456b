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
// One block per entry, one thread per feature pair (2t, 2t+1): the pair is a rotary pair, and
// consecutive threads read consecutive 4-byte (bf16) or 8-byte (fp32) pairs of a token row, so
// every position's loads coalesce.  The kernel is HBM-bound: it reads coff * D * 2 projections per
// token once and writes one cache row per entry.
#include "csa_device.h"
#include "csa_internal.h"

namespace csa {

__device__ __forceinline__ v2f load_pair(const void* base, bool bf16, int64_t off) {
  if (bf16) {
    const uint32_t w = *(const uint32_t*)((const uint16_t*)base + off);
    return v2f{bf16_bits_to_f32(w & 0xFFFFu), bf16_bits_to_f32(w >> 16)};
  }
  return *(const v2f*)((const float*)base + off);
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

template <int D>
__global__ __launch_bounds__(D / 2) void compress_kernel(CompressArgs a) {
  constexpr int NT = D / 2;
  constexpr int kRope = 64;
  const int t = threadIdx.x;
  const int64_t c = a.c_begin + blockIdx.x;
  const bool overlap = a.ratio == 4;
  const int coff = overlap ? 2 : 1;
  const bool bf16 = a.proj_dt == 1;

  // online softmax over the window positions, per feature
  float m0 = -INFINITY, m1 = -INFINITY, l0 = 0.f, l1 = 0.f, s0 = 0.f, s1 = 0.f;
  auto add = [&](int64_t tok, int half, int wpos) {
    const int col = half * D + 2 * t;
    const int64_t off = (tok - a.tok0) * a.ld + col;
    const v2f k = load_pair(a.kv, bf16, off);
    v2f s = load_pair(a.score, bf16, off);
    s[0] += a.ape[(int64_t)wpos * coff * D + col];
    s[1] += a.ape[(int64_t)wpos * coff * D + col + 1];
    const float n0 = fmaxf(m0, s[0]), n1 = fmaxf(m1, s[1]);
    const float r0 = exp2f((m0 - n0) * kLog2e), r1 = exp2f((m1 - n1) * kLog2e);
    const float e0 = exp2f((s[0] - n0) * kLog2e), e1 = exp2f((s[1] - n1) * kLog2e);
    l0 = fmaf(l0, r0, e0);
    l1 = fmaf(l1, r1, e1);
    s0 = fmaf(s0, r0, e0 * k[0]);
    s1 = fmaf(s1, r1, e1 * k[1]);
    m0 = n0;
    m1 = n1;
  };
  if (overlap && c > 0) {
#pragma unroll
    for (int w = 0; w < 4; ++w) add((c - 1) * 4 + w, 0, w);
  }
#pragma unroll 8
  for (int w = 0; w < a.ratio; ++w) add(c * a.ratio + w, overlap ? 1 : 0, w);
  float y0 = s0 / l0, y1 = s1 / l1;

  // RMSNorm over the D features
  __shared__ float red[NT / 64 > 0 ? NT / 64 : 1];
  float ss = wave_sum(y0 * y0 + y1 * y1);
  if constexpr (NT > 64) {
    if ((t & 63) == 0) red[t >> 6] = ss;
    __syncthreads();
    ss = 0.f;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) ss += red[w];
  }
  const float inv = 1.f / sqrtf(ss / (float)D + a.eps);
  y0 = y0 * inv * a.norm_w[2 * t];
  y1 = y1 * inv * a.norm_w[2 * t + 1];

  // rotary embedding of the last 64 features: pair (2t, 2t+1) times cos + i sin
  if (2 * t >= D - kRope) {
    const int p = t - (D - kRope) / 2;
    const float cs = a.rope_cos[(int64_t)blockIdx.x * (kRope / 2) + p];
    const float sn = a.rope_sin[(int64_t)blockIdx.x * (kRope / 2) + p];
    const float r0 = y0 * cs - y1 * sn, r1 = y0 * sn + y1 * cs;
    y0 = r0;
    y1 = r1;
  }

  const int pid = a.page_table[c >> 6];
  const bool mapped = (unsigned)pid < (unsigned)a.num_pages;
  const int64_t slot_row = (int64_t)pid * kPage + (c & (kPage - 1));

  if constexpr (D == 512) {
    uint8_t* row = a.out + slot_row * row_bytes(a.out_fmt);
    if (a.out_fmt == kRowF32) {
      if (mapped) *(v2f*)(row + 8 * t) = v2f{y0, y1};
    } else if (a.out_fmt == kRowBF16) {
      if (mapped) *(uint32_t*)(row + 4 * t) = pack_bf16x2(y0, y1);
    } else if (2 * t < kNope) {
      // e4m3fn nope with one fp32 scale per 64 features (32 threads, lane-aligned halves of a wave)
      float amax = fmaxf(fabsf(y0), fabsf(y1));
#pragma unroll
      for (int m = 1; m < 32; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
      const float sc = fmaxf(amax, 1e-4f) * (1.f / 448.f);
      const int codes = __builtin_amdgcn_cvt_pk_fp8_f32(y0 / sc, y1 / sc, 0, false);
      if (mapped) {
        *(uint16_t*)(row + 2 * t) = (uint16_t)(codes & 0xFFFF);
        if ((t & 31) == 0) *(float*)(row + 576 + 4 * (t >> 5)) = sc;
      }
    } else {
      if (mapped) {
        *(uint32_t*)(row + 448 + 2 * (2 * t - kNope)) = pack_bf16x2(y0, y1);
        if (t == NT - 1) *(uint32_t*)(row + 604) = 0u;
      }
    }
  } else {
    // indexer key: Hadamard rotation over the 128 features (one wave; the butterfly of stride h
    // pairs feature e with e ^ h: within the thread for h = 1, else lane t ^ (h / 2)), then E8M0
    // per 32 features (16 threads) and FP8 or FP4 codes
#pragma unroll
    for (int h = 1; h < D; h <<= 1) {
      if (h == 1) {
        const float u = y0 + y1, v = y0 - y1;
        y0 = u;
        y1 = v;
      } else {
        const float o0 = __shfl_xor(y0, h >> 1), o1 = __shfl_xor(y1, h >> 1);
        const bool hi = (t & (h >> 1)) != 0;
        y0 = hi ? o0 - y0 : y0 + o0;
        y1 = hi ? o1 - y1 : y1 + o1;
      }
    }
    const float hs = 0.08838834764831845f;   // 128^-1/2
    y0 *= hs;
    y1 *= hs;
    float amax = fmaxf(fabsf(y0), fabsf(y1));
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
    const bool fp4 = a.out_fmt == 3;
    const uint32_t e = fp4 ? e8m0_ceil(fmaxf(amax, 6.f * 1.17549435e-38f) / 6.f)
                           : e8m0_ceil(fmaxf(amax, 1e-4f) * (1.f / 448.f));
    const float q = __uint_as_float((254u - e) << 23);   // 2^-(e-127), exact
    if (mapped) {
      if (fp4) {
        a.out[slot_row * 64 + t] = (uint8_t)(e2m1_code(y0 * q) | (e2m1_code(y1 * q) << 4));
      } else {
        const int codes = __builtin_amdgcn_cvt_pk_fp8_f32(y0 * q, y1 * q, 0, false);
        *(uint16_t*)(a.out + slot_row * 128 + 2 * t) = (uint16_t)(codes & 0xFFFF);
      }
      if ((t & 15) == 0) a.out_scales[(int64_t)pid * 256 + (t >> 4) * kPage + (c & (kPage - 1))] = (uint8_t)e;
    }
  }
}

hipError_t launch_compress(const CompressArgs& a, hipStream_t s) {
  if (a.c_count <= 0) return hipSuccess;
  ProfScope p(a.D == 512 ? "compress_kv" : "compress_keys", s);
  if (a.D == 512) hipLaunchKernelGGL(compress_kernel<512>, dim3((unsigned)a.c_count), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(compress_kernel<128>, dim3((unsigned)a.c_count), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace csa
