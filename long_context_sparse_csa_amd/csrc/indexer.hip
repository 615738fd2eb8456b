// C4 indexer scores on gfx950.
//
// Score of compressed entry c for one query ([P1] "DeepSeek-V4 全面解读" section 2.10, forward steps
// 5-8; [P2] "DeepSeek-V4 in SGLang 深度理解分析" concept 3 / algorithm 2):
//     s[c] = sum_h w[h] * max(0, qI[h] . kI[c])
// with FP8 E4M3FN operands that carry one E8M0 scale per 32 elements.
//
// FP8 path: one v_mfma_scale_f32_16x16x128_f8f6f4 covers 16 heads x 16 entries x all 128 dims, and
// its per-lane E8M0 scale operands are exactly the stored per-32 block scales, so dequantisation
// costs nothing.  Operand layout (measured on gfx950): lane l = m + 16*g holds row m, bytes 0..15
// -> k in [16g, 16g+16), bytes 16..31 -> k in [64+16g, 64+16g+16); its scale byte scales row m's
// 32-element block g.  A wave scores one page (64 entries) per step: MFMA column n of key group kg
// is slot 4n+kg, so lane l's scale dword is word l of the page's [4 blocks][64 slots] scale array
// and the key group picks the byte (opsel).  The epilogue applies ReLU and the head weights, then a
// 2-step reduce-scatter over the four lane groups leaves lane l with the full score of slot
// 4*(l%16) + l/16.  Keys stream straight from HBM into VGPRs (no LDS): each lane loads 2 x 16 B per
// key group, and each page is read exactly once.
#include <cstdlib>

#include "csa_device.h"
#include "csa_internal.h"

namespace csa {

template <int HG, int KG>
__device__ __forceinline__ v4f mma_fp8_scaled(const v8i& a, const v8i& b, int sa, int sb, v4f c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, HG, sa, KG, sb);
}

// max(x, 0) in one v_med3_f32 (MFMA results are never signalling NaNs, so no canonicalisation)
__device__ __forceinline__ float relu(float x) { return __builtin_amdgcn_fmed3f(x, 0.f, INFINITY); }

__device__ __forceinline__ v8i load_k_operand(const uint8_t* row, int g) {
  uint4 lo = *(const uint4*)(row + 16 * g);
  uint4 hi = *(const uint4*)(row + 64 + 16 * g);
  v8i r;
  r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
  r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
  return r;
}

__device__ __forceinline__ int64_t visible_count(const IndexerArgs& a, int q, int& r) {
  int64_t nv;
  if (a.vis_mode == 1) {
    r = q;
    int64_t T = a.ctx_len[q];
    nv = (T < 0 ? 0 : (T > a.max_ctx ? a.max_ctx : T)) / 4;
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

// Pages (64 entries each) scored by one wave.  Measured on the batched and long-context decode
// workloads: 2 pages per wave is 15% slower than 4; 8 matches 4 on the first and is 4% faster on
// the second.
constexpr int kPagesPerWave = 8;

template <int NHG, bool HIST>
__global__ __launch_bounds__(256) void indexer_fp8_kernel(IndexerArgs a) {
  constexpr int pages_per_wave = kPagesPerWave;
  const int q = blockIdx.x;   // queries vary fastest: a row's blocks share one XCD (and its L2)
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
  __shared__ uint32_t lhist[HIST ? kHistBins : 1];

  const int64_t c_begin = (int64_t)blockIdx.y * 4 * pages_per_wave * kPage;
  if (c_begin >= a.max_n_vis) return;
  int r;
  const int64_t nv = visible_count(a, q, r);
  if constexpr (HIST) {
    for (int i = tid; i < kHistBins; i += 256) lhist[i] = 0u;
  }

  // A operand: the query's indexer heads, resident in VGPRs.  Loads are unconditional (clamped
  // addresses, padded heads zeroed by select) so nothing waits before the first key page.
  const uint8_t* qb = (const uint8_t*)a.qI + (int64_t)q * a.HI * kDI;
  v8i qa[NHG];
  int qsc = 0;
  float wv[NHG][4];
#pragma unroll
  for (int hg = 0; hg < NHG; ++hg) {
    const int h = 16 * hg + n;
    const int hc = h < a.HI ? h : a.HI - 1;
    const v8i v = load_k_operand(qb + hc * kDI, g);
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

  const uint8_t* keys = (const uint8_t*)a.keys;
  const int32_t* pt = a.page_table + (int64_t)(r < 0 ? 0 : r) * a.max_pages;
  float* lrow = a.logits + (int64_t)q * a.ld;
  const int64_t p_first = (c_begin >> 6) + (int64_t)wave * pages_per_wave;   // this wave's first page
  const int64_t vis_pages = (nv + kPage - 1) / kPage;

  // page ids of this wave's pages, one per lane, then broadcast as needed
  int my_pid = -1;
  {
    const int64_t pp = p_first + lane;
    if (lane < pages_per_wave && pp < vis_pages) my_pid = pt[pp];
  }

  // key page p -> operands; invalid pages read page 0 (always mapped memory) and are masked later
  auto page_ok = [&](int i) {
    const int pid = __shfl(my_pid, i);
    return (unsigned)pid < (unsigned)a.num_pages;
  };
  auto load_page = [&](int i, v8i* kb, int& ksc) {
    int pid = __shfl(my_pid, i);
    pid = (unsigned)pid < (unsigned)a.num_pages ? pid : 0;
    const uint8_t* kp = keys + (int64_t)pid * (kPage * kDI);
    ksc = *(const int*)(a.kscale + (int64_t)pid * 256 + 4 * lane);
#pragma unroll
    for (int kg = 0; kg < 4; ++kg) kb[kg] = load_k_operand(kp + (4 * n + kg) * kDI, g);
  };

  auto compute_page = [&](int i, const v8i* kb, int ksc) {
    const int64_t c0 = (p_first + i) * kPage;
    const bool live = c0 < nv && page_ok(i);
    v4f acc[NHG][4];
    static_for<0, NHG>::run([&](auto HGc) {
      constexpr int HG = decltype(HGc)::value;
      static_for<0, 4>::run([&](auto KGc) {
        constexpr int KG = decltype(KGc)::value;
        acc[HG][KG] = mma_fp8_scaled<HG, KG>(qa[HG], kb[KG], qsc, ksc, v4f{0.f, 0.f, 0.f, 0.f});
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
    // reduce-scatter over the 4 lane groups: lane (n, g) ends with the score of slot 4n+g
    const bool b5 = (lane & 32) != 0;
    float keep0 = b5 ? part[2] : part[0], keep1 = b5 ? part[3] : part[1];
    const float send0 = b5 ? part[0] : part[2], send1 = b5 ? part[1] : part[3];
    keep0 += __shfl_xor(send0, 32);
    keep1 += __shfl_xor(send1, 32);
    const bool b4 = (lane & 16) != 0;
    const float keep = b4 ? keep1 : keep0, send = b4 ? keep0 : keep1;
    const float score = keep + __shfl_xor(send, 16);
    const int64_t c = c0 + 4 * n + g;
    if (c < a.max_n_vis) {
      const float v = (live && c < nv) ? score : -INFINITY;
      lrow[c] = v;
      if constexpr (HIST) {
        if (c < nv) atomicAdd(&lhist[order_key(v) >> kHistShift], 1u);
      }
    }
  };

  // Three page buffers, straight-line code: the first three pages are loaded up front and page
  // i + 3 as soon as page i is scored, so up to three pages are in flight and every wait is for
  // exactly the page about to be scored.  Pages past the wave's range load page 0 (always mapped)
  // and store nothing.
  v8i kb[3][4];
  int ksc[3] = {0, 0, 0};
#pragma unroll
  for (int i = 0; i < 3 && i < pages_per_wave; ++i) load_page(i, kb[i], ksc[i]);
#pragma unroll
  for (int i = 0; i < pages_per_wave; ++i) {
    compute_page(i, kb[i % 3], ksc[i % 3]);
    if (i + 3 < pages_per_wave) load_page(i + 3, kb[i % 3], ksc[i % 3]);
  }
  if constexpr (HIST) {
    __syncthreads();
    uint32_t* gh = a.hist + (int64_t)q * kHistBins;
    for (int i = tid; i < kHistBins; i += 256) {
      const uint32_t v = lhist[i];
      if (v) atomicAdd(&gh[i], v);
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
  if (a.dt == 0) {
    dim3 grid((unsigned)a.Q, (unsigned)((a.max_n_vis + kPage - 1) / kPage));
    ProfScope p("indexer_f32", s);
    if (hist) hipLaunchKernelGGL(indexer_f32_kernel<true>, grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL(indexer_f32_kernel<false>, grid, dim3(256), 0, s, a);
    return hipGetLastError();
  }
  // kPagesPerWave pages per wave, four waves per block
  const int per_block = 4 * kPagesPerWave * kPage;
  dim3 grid((unsigned)a.Q, (unsigned)((a.max_n_vis + per_block - 1) / per_block));
  const int nhg = (a.HI + 15) / 16;
  ProfScope p("indexer_fp8", s);
#define CSA_IDX_LAUNCH(N)                                                                              \
  if (hist) hipLaunchKernelGGL((indexer_fp8_kernel<N, true>), grid, dim3(256), 0, s, a); \
  else hipLaunchKernelGGL((indexer_fp8_kernel<N, false>), grid, dim3(256), 0, s, a);
  switch (nhg) {
    case 1: CSA_IDX_LAUNCH(1) break;
    case 2: CSA_IDX_LAUNCH(2) break;
    case 3: CSA_IDX_LAUNCH(3) break;
    default: CSA_IDX_LAUNCH(4) break;
  }
#undef CSA_IDX_LAUNCH
  return hipGetLastError();
}

}  // namespace csa
