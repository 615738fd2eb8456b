// Device helpers shared by the attention kernels (gather codes, row chunks, matrix-core and
// transposing-LDS wrappers); each translation unit that includes it gets its own zero row.
#pragma once
#include "csa_device.h"
#include "csa_internal.h"

namespace csa {

constexpr int kKrStride = 528;   // bf16 per row of the row-major tile (1056 B, 16-B aligned)
constexpr float kRescaleLog2 = 8.f;

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

// Slot codes: the absolute address of the slot's row (rows are 16-B aligned) with bit 1 set for a
// compressed row (the row format follows from that bit and the kernel's template arguments).
// Invalid slots get the address of kZeroRow, which dequantises to zeros, so V needs no masking; a
// 32-bit mask per tile marks the valid slots for the scores.
typedef const __attribute__((address_space(1))) uint8_t* gbytes;
constexpr uint64_t kCodeComp = 2;
constexpr uint64_t kCodeAddrMask = ~(uint64_t)15;

static __device__ __attribute__((aligned(256))) const uint8_t kZeroRow[1024] = {};

// Codes of four slots of query q (absolute slot indices s[k]; in[k] = the slot exists): all index
// loads, then all page-table loads, are issued before any is used.  ok[k] = the slot has a row.
// idx_list / rows_list, when given, replace the query's row of a.idx (slot-indexed) and of a.rows
// (indexed by compressed slot): a block that selected its own rows keeps them in LDS.
__device__ __forceinline__ void slot_codes4(const AttnArgs& a, int q, int r, const int* s, const bool* in,
                                            uint64_t* code, bool* ok, const int32_t* idx_list = nullptr,
                                            const int32_t* rows_list = nullptr) {
  const bool r_ok = r >= 0 && r < a.n_req;
  const int rr = r_ok ? r : 0;
  const bool has_win = a.win != nullptr;
  const bool has_pt = a.comp != nullptr && a.page_table != nullptr && a.max_pages > 0;
  const int64_t n_entries = (int64_t)a.max_pages * kPage;
  const int32_t* idx_row = idx_list ? idx_list : a.idx + (int64_t)q * a.ld_idx;
  const int32_t* rows_row = rows_list ? rows_list : (a.rows ? a.rows + (int64_t)q * a.ld_rows : nullptr);
  const bool rows_in = rows_row != nullptr && a.comp != nullptr;   // compressed rows arrive resolved
  const uint64_t zero = (uint64_t)(uintptr_t)kZeroRow;
  const int64_t win_rb = row_bytes(a.win_fmt), comp_rb = row_bytes(a.comp_fmt);
  int v[4], pg[4];
  bool live[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    live[k] = r_ok && in[k];
    const int sk = live[k] ? s[k] : 0;
    v[k] = (rows_in && sk >= a.n_win) ? rows_row[sk - a.n_win] : idx_row[sk];
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) pg[k] = -1;
  if (has_pt && !rows_in) {
    const int32_t* pt_row = a.page_table + (int64_t)rr * a.max_pages;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const bool pv = live[k] && s[k] >= a.n_win && v[k] >= 0 && v[k] < n_entries;
      pg[k] = pt_row[pv ? (v[k] >> 6) : 0];
    }
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint64_t c = zero;
    bool o = false;
    if (live[k] && v[k] >= 0) {
      if (s[k] < a.n_win) {
        o = has_win && v[k] < a.win_rows_per_req;
        if (o) c = (uint64_t)(uintptr_t)(a.win + ((int64_t)rr * a.win_rows_per_req + v[k]) * win_rb);
      } else if (rows_in) {
        o = (int64_t)v[k] < (int64_t)a.comp_num_pages * kPage;
        if (o) c = (uint64_t)(uintptr_t)(a.comp + (int64_t)v[k] * comp_rb) | kCodeComp;
      } else {
        o = has_pt && v[k] < n_entries && (unsigned)pg[k] < (unsigned)a.comp_num_pages;
        if (o) c = (uint64_t)(uintptr_t)(a.comp + ((int64_t)pg[k] * kPage + (v[k] & 63)) * comp_rb) | kCodeComp;
      }
      CSA_DBG_COUNT(!o);   // an index that is not -1 yet has no row
    }
    code[k] = c;
    ok[k] = o;
  }
}

// Slots [s_begin, s_begin + s_count) of query q are resolved into `codes` and `vmask` by NT
// threads, four per thread per pass.  s_count is a whole number of tiles, and each wave covers 64
// consecutive slots per pass.
template <int NT>
__device__ __forceinline__ void resolve_codes(const AttnArgs& a, int q, int r, int s_begin, int s_count,
                                              uint64_t* codes, uint32_t* vmask, int tid,
                                              const int32_t* idx_list = nullptr, const int32_t* rows_list = nullptr) {
  const int n_idx = a.n_win + a.n_comp;
  for (int b = 0; b < s_count; b += 4 * NT) {
    int sl[4];
    bool in[4], ok[4];
    uint64_t c[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int i = b + tid + NT * k;
      sl[k] = s_begin + i;
      in[k] = i < s_count && s_begin + i < n_idx;
    }
    slot_codes4(a, q, r, sl, in, c, ok, idx_list, rows_list);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int i = b + tid + NT * k;
      const uint64_t bal = __ballot(ok[k]);
      const int i0 = b + NT * k + (tid & ~63);   // first slot of this wave's 64 (two tiles)
      if (i < s_count) codes[i] = c[k];
      if ((tid & 63) == 0 && i0 < s_count) {
        vmask[i0 / kTile] = (uint32_t)bal;
        if (i0 + kTile < s_count) vmask[i0 / kTile + 1] = (uint32_t)(bal >> 32);
      }
    }
  }
}

typedef uint32_t v2u __attribute__((ext_vector_type(2)));
typedef const __attribute__((address_space(1))) v2u* gv2u;

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

// ds_read_b64_tr_b16 (gfx950).  Measured lane semantics: inside each group of 16 lanes, lane d
// receives element (d & 3) of the 4-element chunks addressed by lanes d/4, d/4+4, d/4+8, d/4+12.
__device__ __forceinline__ v4s lds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)((__attribute__((address_space(3))) uint16_t*)p));
}

}  // namespace csa
