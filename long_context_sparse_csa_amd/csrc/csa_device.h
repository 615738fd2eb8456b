// Device-side helpers shared by the CSA kernels (gfx950 / CDNA4, wave64).
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "csa_internal.h"

// Launch kernel K on stream S; while profiling is on, the scope P's events are attached to the
// dispatch itself (hipExtLaunchKernelGGL), so they bracket the kernel's execution.
#define CSA_LAUNCH(P, K, GRID, BLOCK, S, ...)                                               \
  do {                                                                                      \
    (P).mark();                                                                             \
    hipExtLaunchKernelGGL(K, GRID, BLOCK, 0, S, (P).ev0, (P).ev1, 0, __VA_ARGS__);          \
  } while (0)

namespace csa {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kD = 512;         // head dim: 448 nope + 64 rope
constexpr int kNope = 448;
constexpr int kDI = 128;        // indexer dim
constexpr int kPage = 64;       // compressed entries per page
constexpr int kWin = 128;       // sliding window
constexpr int kHistBins = 4096; // top-k coarse histogram: top 12 bits of the order key
constexpr int kHistShift = 20;

// Debug builds (-DCSA_DEBUG_CHECKS) count the device-resident values the kernels mask as invalid
// (an index at or past its source, a page id outside the pool) into one counter per translation
// unit, read and cleared by csa_debug_violations; release builds compile the counting away.
#ifdef CSA_DEBUG_CHECKS
static __device__ unsigned long long csa_dbg_violations;
#define CSA_DBG_COUNT(cond)                                     \
  do {                                                          \
    if (cond) atomicAdd(&csa_dbg_violations, 1ull);             \
  } while (0)
#define CSA_DBG_ACCESSOR(NAME)                                                                            \
  uint64_t NAME() {                                                                                       \
    unsigned long long v = 0, z = 0;                                                                      \
    if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(csa_dbg_violations), sizeof v, 0, hipMemcpyDeviceToHost) !=    \
        hipSuccess)                                                                                       \
      return ~0ull;                                                                                       \
    (void)hipMemcpyToSymbol(HIP_SYMBOL(csa_dbg_violations), &z, sizeof z, 0, hipMemcpyHostToDevice);     \
    return v;                                                                                             \
  }
#else
#define CSA_DBG_COUNT(cond) \
  do {                      \
  } while (0)
#define CSA_DBG_ACCESSOR(NAME)
#endif

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -1.0e30f;   // finite running-max start: an all-invalid row yields 0


__host__ __device__ constexpr int row_bytes(int fmt) {
  return fmt == kRowF32 ? 2048 : (fmt == kRowBF16 ? 1024 : 608);
}

// Order-preserving map float -> uint32 (larger float -> larger key).  -0.0 is folded onto +0.0 so
// equal scores tie; NaN maps to 0, below -inf.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (f != f) return 0u;
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// order_key without its NaN test: the same order and ties (-0.0 folds onto +0.0: its negation is
// +0.0's key), four operations instead of seven.  Negative scores map to the negation of their bits
// (order_key's complement plus one), so the keys of [-inf, +inf] span [0x00800000, 0xFF800000]
// and NaNs land outside that range; canonical_key maps them to 0 as order_key does.  For code that
// ranks its own keys only (the one-block selection).
__device__ __forceinline__ uint32_t order_key_raw(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? (0u - u) : (u | 0x80000000u);
}

__device__ __forceinline__ uint32_t canonical_key(uint32_t k) {
  return (k < 0x00800000u || k > 0xFF800000u) ? 0u : k;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);   // v_cvt_pk_bf16_f32: RNE
}

typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// Two floats -> two RNE bf16 in one dword (a single v_cvt_pk_bf16_f32), lo in bits [0,16).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const v2f x = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, v2bf));
}

typedef _Float16 v2h __attribute__((ext_vector_type(2)));

// Two floats -> two RNE fp16 in one dword, lo in bits [0,16); and back.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  const v2f x = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, v2h));
}
__device__ __forceinline__ v2f unpack_f16x2(uint32_t w) {
  return __builtin_convertvector(__builtin_bit_cast(v2h, w), v2f);
}

// 4 e4m3fn bytes of `w` -> 4 floats (hardware conversion, OCP e4m3fn on gfx950).
__device__ __forceinline__ void fp8x4_to_f32(uint32_t w, float* o) {
  v2f a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  v2f b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  o[0] = a[0]; o[1] = a[1]; o[2] = b[0]; o[3] = b[1];
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

// Max / sum over lanes l, l^16, l^32, l^48 (the four 16-lane rows), broadcast to all four, with
// the cross-row lane swaps (v_permlane32_swap: upper half of the first operand <-> lower half of
// the second; v_permlane16_swap: odd rows of the first <-> even rows of the second) instead of
// LDS-routed shuffles.  Swapping a value with itself leaves the two halves (rows) side by side in
// the two results.
__device__ __forceinline__ float row_group_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float row_group_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Largest uint32 over the 64 lanes, with DPP moves inside each 16-lane row (quad permutations
// for strides 1 and 2, row rotations for 4 and 8) and the cross-row lane swaps for 16 and 32: no
// LDS-routed shuffle (a chain of those measured about a microsecond per block-wide reduction).
__device__ __forceinline__ uint32_t wave_umax(uint32_t x) {
  auto mx = [](uint32_t p, uint32_t q) { return p > q ? p : q; };
  x = mx(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xf, 0xf, false));   // quad_perm 1,0,3,2
  x = mx(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xf, 0xf, false));   // quad_perm 2,3,0,1
  x = mx(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x124, 0xf, 0xf, false));  // row_ror:4
  x = mx(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x128, 0xf, 0xf, false));  // row_ror:8
  auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = mx(r[0], r[1]);
  r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return mx(r[0], r[1]);
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves (VALU only, no LDS crossbar):
// shifts by 1, 2, 4, 8 inside each row of 16 lanes, then row 0's and row 2's totals broadcast into
// rows 1 and 3, then the total of rows 0-1 into rows 2 and 3.  Lanes without a source add 0.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, true);   // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, true);   // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, true);   // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, true);   // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

// Decode with S queries per request: query q is token j = q % S of request r = q / S, one of the
// last S tokens of that request's T = ctx_len[r] (clamped to [0, max_ctx]); it sits at position
// T - S + j and sees the T - (S - 1 - j) tokens up to it (0 if that is negative).
// Ring slot of decode position p >= 0 (32-bit division when p fits, as it does for any context a
// ring serves; a 64-bit division is some 50 instructions).
__device__ __forceinline__ int32_t ring_slot(int64_t p, int ring) {
  return p <= 0x7FFFFFFF ? (int32_t)((uint32_t)p % (uint32_t)ring) : (int32_t)(p % ring);
}

// decode_seen_of takes T = ctx_len[q / S] already loaded.
__device__ __forceinline__ int64_t decode_seen_of(int64_t T, int64_t max_ctx, int S, int q) {
  T = T < 0 ? 0 : (T > max_ctx ? max_ctx : T);
  T -= S - 1 - (q - (q / S) * S);
  return T < 0 ? 0 : T;
}

__device__ __forceinline__ int64_t decode_seen(const int32_t* ctx_len, int64_t max_ctx, int S, int q, int& r) {
  r = q / S;
  return decode_seen_of(ctx_len[r], max_ctx, S, q);
}

template <int I, int N>
struct static_for {
  template <class F>
  __device__ __forceinline__ static void run(F&& f) {
    if constexpr (I < N) {
      f(std::integral_constant<int, I>{});
      static_for<I + 1, N>::run(f);
    }
  }
};

}  // namespace csa
