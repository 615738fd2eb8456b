// Index-gathered multi-query attention with a per-head sink on gfx950.
//
// What is computed follows [P1] "DeepSeek-V4 全面解读" section 3.7 (sparse_attn_kernel): rows are
// gathered by index, -1 slots are masked, scores are scale * q.kv, an online softmax keeps a running
// max and sum, P.V accumulates, and after the loop e^(sink - max) joins the denominator.  [P3]
// "tilelang量化内核拆解…" (sparse_attn section) fixes the running-max start at the finite -1e30, so a
// query with no valid slot outputs exact zeros.  K and V are the same 512-dim rows.
//
// BF16 matrix-core kernel (q bf16): a block owns one query, up to 64 heads (one wave per 16 heads)
// and a contiguous range of 32-slot tiles.  Per tile the block gathers the 32 rows once (coalesced:
// one 16-B lane chunk per 8 dims of a row, FP8 nope dequantised with its fp32 block scale), writes
// them to LDS twice as bf16 - row-major for S^T = K.q^T and transposed for O^T = V^T.P^T - and each
// wave runs 2x16 + 32 v_mfma_f32_16x16x32_bf16.  Computing S transposed leaves each lane holding 8
// scores of its own head, which are exactly the P^T operand of the P.V product once the key order
// inside the 32-wide K step is permuted (slot 8g+4mt+i <-> key 16mt+4g+i); the transposed V tile is
// written in that slot order.  Softmax runs in base 2 with log2(e) folded into the scale.
// Large queries-by-heads grids run unsplit; small ones split the slot range across blocks and a
// combine kernel merges the (max, sum, acc) partials, sink included.
//
// fp32 kernel (q f32): one block per (query, head); scores, softmax and P.V in fp32 with natural
// exp, for bit-accurate-ish comparisons against the fp64 definition.
#include "csa_device.h"
#include "csa_internal.h"

namespace csa {

constexpr int kTile = 32;
constexpr int kKrStride = 520;   // bf16 per row of the row-major tile (1040 B, 16-B aligned)
constexpr int kVtStride = 36;    // bf16 per row of the transposed tile (72 B)
constexpr int kMaxSplit = 8;

struct RowSrc {
  const uint8_t* p;
  int fmt;
};

// Resolve slot s of query q's index list to a row address (nullptr = invalid slot).
__device__ __forceinline__ RowSrc resolve_slot(const AttnArgs& a, int q, int r, int s) {
  RowSrc rs{nullptr, 0};
  if (r < 0 || r >= a.n_req || s >= a.n_win + a.n_comp) return rs;
  const int v = a.idx[(int64_t)q * a.ld_idx + s];
  if (v < 0) return rs;
  if (s < a.n_win) {
    if (a.win != nullptr && v < a.win_rows_per_req) {
      rs.p = a.win + ((int64_t)r * a.win_rows_per_req + v) * row_bytes(a.win_fmt);
      rs.fmt = a.win_fmt;
    }
  } else if (a.comp != nullptr && (int64_t)v < (int64_t)a.max_pages * kPage) {
    const int pg = a.page_table[(int64_t)r * a.max_pages + (v >> 6)];
    if ((unsigned)pg < (unsigned)a.comp_num_pages) {
      rs.p = a.comp + ((int64_t)pg * kPage + (v & 63)) * row_bytes(a.comp_fmt);
      rs.fmt = a.comp_fmt;
    }
  }
  return rs;
}

// Dims [8*dc, 8*dc+8) of a row, dequantised to fp32.
__device__ __forceinline__ void load_chunk8(const uint8_t* row, int fmt, int dc, float* v) {
  if (row == nullptr) {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = 0.f;
    return;
  }
  if (fmt == kRowBF16) {
    const uint4 x = *(const uint4*)(row + 16 * dc);
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = __uint_as_float(w[e] << 16);
      v[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
    }
  } else if (fmt == kRowF32) {
    const float4 x = *(const float4*)(row + 32 * dc);
    const float4 y = *(const float4*)(row + 32 * dc + 16);
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
    v[4] = y.x; v[5] = y.y; v[6] = y.z; v[7] = y.w;
  } else if (dc < kNope / 8) {
    const uint2 x = *(const uint2*)(row + 8 * dc);
    const float sc = *(const float*)(row + 576 + 4 * (dc >> 3));
    fp8x4_to_f32(x.x, v);
    fp8x4_to_f32(x.y, v + 4);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] *= sc;
  } else {
    const uint4 x = *(const uint4*)(row + 448 + 16 * (dc - kNope / 8));
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = __uint_as_float(w[e] << 16);
      v[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
    }
  }
}

__device__ __forceinline__ v4f mma_bf16(const v8bf& a, const v8bf& b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void store4(void* out, int out_dt, int64_t off, float a0, float a1, float a2, float a3) {
  if (out_dt == 0) {
    *(float4*)((float*)out + off) = make_float4(a0, a1, a2, a3);
  } else {
    *(uint2*)((uint16_t*)out + off) = make_uint2(pack_bf16x2(a0, a1), pack_bf16x2(a2, a3));
  }
}

__global__ __launch_bounds__(256, 1) void attn_bf16_kernel(AttnArgs a) {
  const int nw = blockDim.x >> 6;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int q = blockIdx.x / a.n_split, split = blockIdx.x % a.n_split;
  const int Hpad = (a.H + 15) & ~15;
  const int h = blockIdx.y * 64 + wave * 16 + n;   // this lane's head
  const bool h_ok = h < a.H;

  __shared__ __align__(16) uint16_t Kr[kTile * kKrStride];
  __shared__ __align__(16) uint16_t Vt[kD * kVtStride];
  __shared__ const uint8_t* rowp[kTile];
  __shared__ int rowf[kTile];
  __shared__ int nvalid;

  const int n_idx = a.n_win + a.n_comp;
  const int n_tiles = (n_idx + kTile - 1) / kTile;
  const int tps = (n_tiles + a.n_split - 1) / a.n_split;
  const int t_begin = split * tps;
  const int t_end = min(n_tiles, t_begin + tps);
  const int r = a.q_req[q];

  // q^T operand: lane holds q[h][32ks + 8g .. +8] for the 16 K-steps of 32 dims
  v8bf qf[16];
  {
    const uint16_t* qrow = (const uint16_t*)a.q + ((int64_t)q * a.H + (h_ok ? h : 0)) * kD;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      if (h_ok) {
        qf[ks] = *(const v8bf*)(qrow + 32 * ks + 8 * g);
      } else {
        qf[ks] = v8bf{};
      }
    }
  }

  const float sc = a.softmax_scale * kLog2e;
  float m = kNegBig, lsum = 0.f;
  v4f acc[32];
#pragma unroll
  for (int dt = 0; dt < 32; ++dt) acc[dt] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int t = t_begin; t < t_end; ++t) {
    __syncthreads();
    RowSrc rs{nullptr, 0};
    if (tid < kTile) {
      rs = resolve_slot(a, q, r, t * kTile + tid);
      rowp[tid] = rs.p;
      rowf[tid] = rs.fmt;
    }
    if (wave == 0) {
      const unsigned long long b = __ballot(tid < kTile && rs.p != nullptr);
      if (lane == 0) nvalid = __popcll(b);
    }
    __syncthreads();
    if (nvalid == 0) continue;

    // gather: rows (2pr, 2pr+1), lane = dim chunk; bf16 into Kr (row-major) and Vt (transposed)
    for (int pr = wave; pr < kTile / 2; pr += nw) {
      const int j0 = 2 * pr;
      float v0[8], v1[8];
      load_chunk8(rowp[j0], rowf[j0], lane, v0);
      load_chunk8(rowp[j0 + 1], rowf[j0 + 1], lane, v1);
      uint32_t w0[4], w1[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        w0[e] = pack_bf16x2(v0[2 * e], v0[2 * e + 1]);
        w1[e] = pack_bf16x2(v1[2 * e], v1[2 * e + 1]);
      }
      *(uint4*)&Kr[j0 * kKrStride + 8 * lane] = make_uint4(w0[0], w0[1], w0[2], w0[3]);
      *(uint4*)&Kr[(j0 + 1) * kKrStride + 8 * lane] = make_uint4(w1[0], w1[1], w1[2], w1[3]);
      const int slot = 8 * ((j0 & 15) >> 2) + 4 * (j0 >> 4) + (j0 & 3);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t lo = (w0[e] & 0xFFFFu) | (w1[e] << 16);      // dim 8*lane + 2e
        const uint32_t hi = (w0[e] >> 16) | (w1[e] & 0xFFFF0000u);  // dim 8*lane + 2e + 1
        *(uint32_t*)&Vt[(8 * lane + 2 * e) * kVtStride + slot] = lo;
        *(uint32_t*)&Vt[(8 * lane + 2 * e + 1) * kVtStride + slot] = hi;
      }
    }
    __syncthreads();

    // S^T[key][head] for keys 0..15 (s0) and 16..31 (s1)
    v4f s0 = v4f{0.f, 0.f, 0.f, 0.f}, s1 = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      const v8bf k0 = *(const v8bf*)&Kr[n * kKrStride + 32 * ks + 8 * g];
      const v8bf k1 = *(const v8bf*)&Kr[(16 + n) * kKrStride + 32 * ks + 8 * g];
      s0 = mma_bf16(k0, qf[ks], s0);
      s1 = mma_bf16(k1, qf[ks], s1);
    }
    float sv[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sv[i] = rowp[4 * g + i] != nullptr ? s0[i] * sc : -INFINITY;
      sv[4 + i] = rowp[16 + 4 * g + i] != nullptr ? s1[i] * sc : -INFINITY;
    }
    float tmax = sv[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) tmax = fmaxf(tmax, sv[e]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m, tmax);
    const float alpha = exp2f(m - m_new);
    float p[8], psum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      p[e] = exp2f(sv[e] - m_new);
      psum += p[e];
    }
    lsum = lsum * alpha + psum;
    if (__any(m_new != m)) {
#pragma unroll
      for (int dt = 0; dt < 32; ++dt) acc[dt] *= alpha;
    }
    m = m_new;
    v8bf pf;
#pragma unroll
    for (int e = 0; e < 8; ++e) pf[e] = (__bf16)p[e];

    // O^T[d][head] += V^T[d][slot] . P^T[slot][head]
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) {
      const uint16_t* vp = &Vt[(16 * dt + n) * kVtStride + 8 * g];
      const uint2 lo = *(const uint2*)vp;
      const uint2 hi = *(const uint2*)(vp + 4);
      const uint4 vv = make_uint4(lo.x, lo.y, hi.x, hi.y);
      acc[dt] = mma_bf16(__builtin_bit_cast(v8bf, vv), pf, acc[dt]);
    }
  }

  float ltot = lsum + __shfl_xor(lsum, 16);
  ltot += __shfl_xor(ltot, 32);
  if (a.n_split == 1) {
    if (!h_ok) return;
    const float sk = a.sink[h] * kLog2e;
    const float M = fmaxf(m, sk);
    const float f = exp2f(m - M);
    const float inv = f / (ltot * f + exp2f(sk - M));
    const int64_t ob = ((int64_t)q * a.H + h) * kD;
#pragma unroll
    for (int dt = 0; dt < 32; ++dt)
      store4(a.out, a.out_dt, ob + 16 * dt + 4 * g, acc[dt][0] * inv, acc[dt][1] * inv, acc[dt][2] * inv,
             acc[dt][3] * inv);
  } else {
    if (h >= Hpad) return;
    const int64_t prow = ((int64_t)q * a.n_split + split) * Hpad + h;
    float* pa = a.part + prow * kD;
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) *(float4*)(pa + 16 * dt + 4 * g) = make_float4(acc[dt][0], acc[dt][1], acc[dt][2], acc[dt][3]);
    float* pml = a.part + (int64_t)a.Q * a.n_split * Hpad * kD + prow * 2;
    if (g == 0) {
      pml[0] = m;
      pml[1] = ltot;
    }
  }
}

// Merge split-K partials: out = sum_s acc_s 2^(m_s-M) / (sum_s l_s 2^(m_s-M) + 2^(sink-M)).
__global__ __launch_bounds__(128) void attn_combine_kernel(AttnArgs a) {
  const int q = blockIdx.x / a.H, h = blockIdx.x % a.H;
  const int Hpad = (a.H + 15) & ~15;
  const float* ml = a.part + (int64_t)a.Q * a.n_split * Hpad * kD;
  const float sk = a.sink[h] * kLog2e;
  float M = sk;
  for (int s = 0; s < a.n_split; ++s) M = fmaxf(M, ml[(((int64_t)q * a.n_split + s) * Hpad + h) * 2]);
  float den = exp2f(sk - M);
  float w[kMaxSplit];
  for (int s = 0; s < a.n_split; ++s) {
    const int64_t prow = ((int64_t)q * a.n_split + s) * Hpad + h;
    w[s] = exp2f(ml[prow * 2] - M);
    den += w[s] * ml[prow * 2 + 1];
  }
  const float inv = 1.f / den;
  const int d = threadIdx.x * 4;
  float o[4] = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < a.n_split; ++s) {
    const int64_t prow = ((int64_t)q * a.n_split + s) * Hpad + h;
    const float4 x = *(const float4*)(a.part + prow * kD + d);
    o[0] = fmaf(w[s], x.x, o[0]);
    o[1] = fmaf(w[s], x.y, o[1]);
    o[2] = fmaf(w[s], x.z, o[2]);
    o[3] = fmaf(w[s], x.w, o[3]);
  }
  store4(a.out, a.out_dt, ((int64_t)q * a.H + h) * kD + d, o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv);
}

// fp32 path: block = (query, head); all arithmetic in fp32.
__global__ __launch_bounds__(256) void attn_f32_kernel(AttnArgs a) {
  const int q = blockIdx.x, h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ float S[4096];
  __shared__ float red[4 * kD];
  __shared__ float s_stat[4];
  const int n_idx = a.n_win + a.n_comp;
  const int r = a.q_req[q];
  const float* qrow = (const float*)a.q + ((int64_t)q * a.H + h) * kD;
  float qv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) qv[e] = qrow[8 * lane + e];

  float lmax = -INFINITY;
  for (int j = wave; j < n_idx; j += 4) {
    const RowSrc rs = resolve_slot(a, q, r, j);
    float s = -INFINITY;
    if (rs.p != nullptr) {
      float v[8];
      load_chunk8(rs.p, rs.fmt, lane, v);
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) d = fmaf(qv[e], v[e], d);
      s = wave_sum(d) * a.softmax_scale;
    }
    if (lane == 0) S[j] = s;
    lmax = fmaxf(lmax, s);
  }
  if (lane == 0) s_stat[wave] = lmax;
  __syncthreads();
  const float sink = a.sink[h];
  const float M = fmaxf(fmaxf(fmaxf(s_stat[0], s_stat[1]), fmaxf(s_stat[2], s_stat[3])), sink);
  __syncthreads();
  float lsum = 0.f;
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j = wave; j < n_idx; j += 4) {
    const float s = S[j];
    if (s == -INFINITY) continue;
    const float p = expf(s - M);
    lsum += p;
    const RowSrc rs = resolve_slot(a, q, r, j);
    float v[8];
    load_chunk8(rs.p, rs.fmt, lane, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = fmaf(p, v[e], o[e]);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[wave * kD + 8 * lane + e] = o[e];
  if (lane == 0) s_stat[wave] = lsum;
  __syncthreads();
  const float den = s_stat[0] + s_stat[1] + s_stat[2] + s_stat[3] + expf(sink - M);
  for (int d = tid; d < kD; d += 256) {
    const float x = (red[d] + red[kD + d]) + (red[2 * kD + d] + red[3 * kD + d]);
    const float y = x / den;
    if (a.out_dt == 0) ((float*)a.out)[((int64_t)q * a.H + h) * kD + d] = y;
    else ((uint16_t*)a.out)[((int64_t)q * a.H + h) * kD + d] = (uint16_t)f32_to_bf16_bits(y);
  }
}

int plan_attn_split(int Q, int H, int n_idx, int q_dt) {
  if (q_dt == 0) return 1;
  const int hchunks = (((H + 15) & ~15) + 63) / 64;
  const int n_tiles = (n_idx + kTile - 1) / kTile;
  const int blocks = Q * hchunks;
  int s = (256 + blocks - 1) / blocks;
  const int max_s = n_tiles / 2 > 1 ? n_tiles / 2 : 1;
  if (s > max_s) s = max_s;
  if (s > kMaxSplit) s = kMaxSplit;
  if (s < 1) s = 1;
  return s;
}

size_t attn_partial_bytes(int Q, int H, int n_idx) {
  const int s = plan_attn_split(Q, H, n_idx, 1);
  if (s <= 1) return 0;
  const size_t Hpad = (size_t)((H + 15) & ~15);
  return (size_t)Q * s * Hpad * (kD + 2) * sizeof(float);
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  const int n_idx = a.n_win + a.n_comp;
  if (a.q_dt == 0) {
    ProfScope p("attn_f32", s);
    hipLaunchKernelGGL(attn_f32_kernel, dim3((unsigned)a.Q, (unsigned)a.H), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  const int Hpad = (a.H + 15) & ~15;
  const int hchunks = (Hpad + 63) / 64;
  const int waves = Hpad >= 64 ? 4 : Hpad / 16;
  {
    ProfScope p("attn_bf16", s);
    hipLaunchKernelGGL(attn_bf16_kernel, dim3((unsigned)(a.Q * a.n_split), (unsigned)hchunks), dim3(64 * waves), 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_split == 1) return e;
  (void)n_idx;
  ProfScope p("attn_combine", s);
  hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)(a.Q * a.H)), dim3(128), 0, s, a);
  return hipGetLastError();
}

}  // namespace csa
