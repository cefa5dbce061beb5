// Helpers shared by the expert FFN kernels (weight formats, work units,
// streaming loads).  See expert_decode.hip for the arithmetic.
#pragma once

#include <math.h>

#include "common.h"

namespace moe {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kGuRows = 8;        // rows staged per pass of the gate/up kernel
constexpr int kDnRows = 16;       // rows staged per pass of the down kernel
constexpr int kGuSlice = 8;       // gate/up rows (f) per item: 8 gate + 8 up rows
constexpr int kDnSlice = 64;      // down rows (h) per item
constexpr int kSharedChunk = 64;  // shared-expert rows per item
constexpr int kGuStageItems = 2;  // (row, chunk) activation pieces a thread loads before staging them

// 16-byte streaming load (weights are read once).
MOE_DEV uint4 load_stream16(const uint4 *p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// byte n of w as float (v_cvt_f32_ubyte<n>)
template <int N>
MOE_DEV float ubyte_f32(uint32_t w) {
  return static_cast<float>((w >> (8 * N)) & 0xFFu);
}

MOE_DEV float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                         false);
}

template <int FMT>
struct FmtTraits;
template <>
struct FmtTraits<MOE_W_INT8_ROW> {
  static constexpr int kElemsPerChunk = 16;
  static constexpr int kXDwordsPerChunk = 8;   // staged bf16 pairs per chunk
  static constexpr float kOffset = 128.f;      // stored value = q + 128
  static constexpr int kRowBytesPerElem2 = 2;  // row bytes = Kin * this / 2
};
template <>
struct FmtTraits<MOE_W_INT4_B32> {
  static constexpr int kElemsPerChunk = 32;
  static constexpr int kXDwordsPerChunk = 16;
  static constexpr float kOffset = 136.f;  // bf16 magic value = q + 136
  static constexpr int kRowBytesPerElem2 = 1;
};

// One unit of work: an expert's weights and a range of its rows.
struct Unit {
  const void *gq, *gs, *uq, *us, *dq, *ds;
  int F;      // SwiGLU width of this expert
  int e;      // expert index inside its arrays
  int r0, n;  // rows [r0, r0 + n) of the unit
  bool shared;
};

// Row r of a unit: its token, its act row offset (floats), its output row
// and its routing weight.
MOE_DEV int unit_token(const FfnArgs &a, const Unit &u, int r) {
  if (u.shared) return r;
  return a.row_tok ? a.row_tok[r] : r;
}
MOE_DEV size_t unit_act_off(const FfnArgs &a, const Unit &u, int r) {
  return u.shared ? static_cast<size_t>(a.n_rows) * a.F + static_cast<size_t>(r) * a.Fs
                  : static_cast<size_t>(r) * a.F;
}
MOE_DEV int unit_out_row(const FfnArgs &a, const Unit &u, int r) { return u.shared ? a.n_rows + r : r; }
MOE_DEV float unit_row_w(const FfnArgs &a, const Unit &u, int r) {
  if (u.shared || !a.row_w) return 1.f;
  return a.row_w[r];
}

MOE_DEV int routed_units(const FfnArgs &a) { return a.offsets ? *a.n_active : (a.n_rows > 0 ? 1 : 0); }
MOE_DEV int shared_chunks(const FfnArgs &a) { return a.Fs > 0 ? (a.T + kSharedChunk - 1) / kSharedChunk : 0; }

// Item i -> (unit, slice).  Routed items first: unit = i / slices; then the
// shared expert's items: (slice, chunk of kSharedChunk rows).
MOE_DEV bool item_unit(const FfnArgs &a, int i, int U, int slices, int slices_sh, Unit &u, int &slice) {
  const int n_routed = U * slices;
  if (i < n_routed) {
    const int k = i / slices;
    slice = i - k * slices;
    u.shared = false;
    u.gq = a.gq;
    u.gs = a.gs;
    u.uq = a.uq;
    u.us = a.us;
    u.dq = a.dq;
    u.ds = a.ds;
    u.F = a.F;
    if (a.offsets) {
      u.e = a.active[k];
      u.r0 = a.offsets[u.e];
      u.n = a.offsets[u.e + 1] - u.r0;
    } else {
      u.e = 0;
      u.r0 = 0;
      u.n = a.n_rows;
    }
    return true;
  }
  const int jj = i - n_routed;
  const int chunk = jj / slices_sh;
  slice = jj - chunk * slices_sh;
  u.shared = true;
  u.gq = a.sgq;
  u.gs = a.sgs;
  u.uq = a.suq;
  u.us = a.sus;
  u.dq = a.sdq;
  u.ds = a.sds;
  u.F = a.Fs;
  u.e = 0;
  u.r0 = chunk * kSharedChunk;
  u.n = min(kSharedChunk, a.T - u.r0);
  return u.n > 0;
}

template <int QUADS>
MOE_DEV int quad_slot(int c, int qd) {
  return (qd + (c >> 2)) & (QUADS - 1);
}

// float4 index inside a staged fp32 row: the eight 16-byte groups of each
// 128-byte chunk c are rotated by c so that lanes reading consecutive chunks
// spread over the LDS banks
MOE_DEV int act_slot(int c, int k) { return c * 8 + ((k + c) & 7); }  // float4 index inside a row

// Launchers: the item kernels (any token count, both formats) and the
// int4 matrix-core kernels for decode batches (act rows as bf16 hi/lo
// planes); gate/up and down must use the same family for one call.
hipError_t launch_gateup_items(const FfnArgs &a, hipStream_t s);
hipError_t launch_down_items(const FfnArgs &a, hipStream_t s);
bool mfma_decode_ok(const FfnArgs &a);
hipError_t launch_gateup_mfma(const FfnArgs &a, hipStream_t s);
hipError_t launch_down_mfma(const FfnArgs &a, hipStream_t s);
bool prefill_ok(const FfnArgs &a);
hipError_t launch_gateup_prefill(const FfnArgs &a, hipStream_t s);
hipError_t launch_down_prefill(const FfnArgs &a, hipStream_t s);

}  // namespace moe
