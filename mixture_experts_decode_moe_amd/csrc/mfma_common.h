// Helpers of the matrix-core expert kernels (bf16 MFMA on exact integer
// operands): operand conversions, the cross-row transpose of weight
// chunks, per-format traits.  The arithmetic is described in
// expert_mfma.hip.
#pragma once

#include <utility>

#include "expert_common.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr uint32_t kMinus136Pair = 0xC308C308u;  // bf16 pair (-136, -136)
constexpr int kGuMaxWaves = 16;  // gate/up: waves splitting the hidden dimension
constexpr int kDnMaxWaves = 8;   // down: waves splitting the SwiGLU dimension

MOE_DEV f32x4_t mfma_bf16(const u32x4_t &a, const u32x4_t &b, const f32x4_t &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                 c, 0, 0, 0);
}

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2v_t __attribute__((ext_vector_type(2)));

// A pair of bf16 (one word) -> the same pair in fp16: exact for magnitudes
// in fp16's normal range [2^-14, 65504], rounded to nearest below it.
MOE_DEV uint32_t bf16x2_to_f16x2(uint32_t u) {
  const f32x2v_t f = {__uint_as_float(u << 16), __uint_as_float(u & 0xFFFF0000u)};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2_t));
}

// Eight nibbles (one k-group of a 32-element block, stored as q + 8) and the
// block's fp16 scale s -> four fp16 pairs (q_i s, q_{i+4} s), i = 0..3, in
// the pair order of magic_pairs: 0x6400 | n is 1024 + n exactly, minus 1032
// gives q exactly, and the product with s is rounded once to fp16 (relative
// error at most 2^-11).  s is scale p (0..3) of a pair of words holding four
// consecutive scales; the packed multiply reads it from its half of the word
// for both lanes of the pair (no separate splat).
MOE_DEV u32x4_t dequant_f16_pairs(uint32_t w, uint32_t s01, uint32_t s23, int p) {
  const uint32_t ev = w & 0x0F0F0F0Fu;
  const uint32_t od = (w >> 4) & 0x0F0F0F0Fu;
  const uint32_t hi = 0x64646464u;
  const uint32_t r[4] = {__builtin_amdgcn_perm(hi, ev, 0x04020400u), __builtin_amdgcn_perm(hi, od, 0x04020400u),
                         __builtin_amdgcn_perm(hi, ev, 0x04030401u), __builtin_amdgcn_perm(hi, od, 0x04030401u)};
  const f16x2_t off = {static_cast<_Float16>(-1032.0f), static_cast<_Float16>(-1032.0f)};
  const f16x2_t sw = __builtin_bit_cast(f16x2_t, p < 2 ? s01 : s23);
  const _Float16 sv = (p & 1) ? sw[1] : sw[0];
  const f16x2_t sc = {sv, sv};
  u32x4_t out;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f16x2_t q = __builtin_bit_cast(f16x2_t, r[i]) + off;  // exact
    out[i] = __builtin_bit_cast(uint32_t, q * sc);
  }
  return out;
}

MOE_DEV f32x4_t mfma_bf16_k16(const u32x2_t &a, const u32x2_t &b, const f32x4_t &c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a), __builtin_bit_cast(s16x4_t, b), c,
                                                   0, 0, 0);
}

// Four int8 weights (one k-group) -> two bf16 pairs of q (exact: |q| <= 127
// needs 7 bits).  Each byte goes through fp32 as its unsigned value of
// byte ^ 0x80 = q + 128 minus 128 (both steps exact; a float conversion of a
// sign-extended field has been miscompiled).
MOE_DEV u32x2_t byte_pairs(uint32_t w) {
  const uint32_t v = w ^ 0x80808080u;
  const float f0 = static_cast<float>(v & 0xFFu) - 128.f, f1 = static_cast<float>((v >> 8) & 0xFFu) - 128.f;
  const float f2 = static_cast<float>((v >> 16) & 0xFFu) - 128.f, f3 = static_cast<float>(v >> 24) - 128.f;
  u32x2_t r;
  r.x = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);  // high halves
  r.y = __builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), 0x07060302u);
  return r;
}

// Eight nibbles (one k-group) -> four bf16 pairs (128 + n_s, 128 + n_{s+4}).
// The even nibbles n0 n2 n4 n6 and the odd ones n1 n3 n5 n7 are split into
// bytes once, then each pair is one byte permute with the 0x43 high bytes:
// seven operations a word.
MOE_DEV u32x4_t magic_pairs(uint32_t w) {
  const uint32_t ev = w & 0x0F0F0F0Fu;
  const uint32_t od = (w >> 4) & 0x0F0F0F0Fu;
  const uint32_t hi = 0x43434343u;
  u32x4_t r;
  r.x = __builtin_amdgcn_perm(hi, ev, 0x04020400u);  // (n0, n4)
  r.y = __builtin_amdgcn_perm(hi, od, 0x04020400u);  // (n1, n5)
  r.z = __builtin_amdgcn_perm(hi, ev, 0x04030401u);  // (n2, n6)
  r.w = __builtin_amdgcn_perm(hi, od, 0x04030401u);  // (n3, n7)
  return r;
}

// Eight consecutive bf16 (four words) -> pairs (x_s, x_{s+4}), s = 0..3.
MOE_DEV u32x4_t pair_permute(const uint4 &d) {
  u32x4_t r;
  r.x = __builtin_amdgcn_perm(d.z, d.x, 0x05040100u);  // low halves of d.x, d.z
  r.y = __builtin_amdgcn_perm(d.z, d.x, 0x07060302u);  // high halves
  r.z = __builtin_amdgcn_perm(d.w, d.y, 0x05040100u);
  r.w = __builtin_amdgcn_perm(d.w, d.y, 0x07060302u);
  return r;
}

// 4x4 transpose of 32-bit values across the four 16-lane rows: afterwards
// register p of row g holds what register g of row p held.
MOE_DEV void xpose4(uint4 &v) {
  const auto a = __builtin_amdgcn_permlane32_swap(v.x, v.z, false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(v.y, v.w, false, false);
  const auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
  const auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
  v = make_uint4(c[0], c[1], d[0], d[1]);
}

MOE_DEV uint32_t word(const uint4 &v, int p) { return p == 0 ? v.x : p == 1 ? v.y : p == 2 ? v.z : v.w; }

// fp16 scale p (0..3) of a pair of words holding four consecutive scales
MOE_DEV float scale4(uint32_t s01, uint32_t s23, int p) {
  const uint32_t w = p < 2 ? s01 : s23;
  return f16_bits_to_f32(static_cast<uint16_t>((p & 1) ? (w >> 16) : (w & 0xFFFFu)));
}

MOE_DEV f32x4_t fma4(float s, const f32x4_t &c, const f32x4_t &acc) {
  f32x4_t r;
  r.x = fmaf(s, c.x, acc.x);
  r.y = fmaf(s, c.y, acc.y);
  r.z = fmaf(s, c.z, acc.z);
  r.w = fmaf(s, c.w, acc.w);
  return r;
}

// Position of SwiGLU column f inside its row of the act planes: the
// element order of the MFMA operands (int4: (f, f + 4) adjacent within each
// group of 8; int8: natural order).
template <int FMT>
MOE_DEV int act_pos(int f) {
  if constexpr (FMT == MOE_W_INT4_B32) return (f & ~7) | ((f & 3) << 1) | ((f >> 2) & 1);
  return f;
}

// Per-format pieces of the MFMA kernels: k per block (one 16-byte chunk of a
// weight row), the A operand from a bf16 row, the B operand from a weight
// k-group word, and the MFMA.
template <int FMT>
struct MfmaFmt;
template <>
struct MfmaFmt<MOE_W_INT4_B32> {
  static constexpr int kBlockK = 32;
  using Vec = u32x4_t;
  // k-group g of block b of a bf16 row, pair-permuted
  static MOE_DEV Vec a_x(const uint16_t *row, int b, int g) {
    return pair_permute(reinterpret_cast<const uint4 *>(row)[4 * b + g]);
  }
  // the same from a hi or lo act plane (already in operand order)
  static MOE_DEV Vec a_plane(const uint16_t *plane, int b, int g) {
    const uint4 v = reinterpret_cast<const uint4 *>(plane)[4 * b + g];
    return Vec{v.x, v.y, v.z, v.w};
  }
  static MOE_DEV Vec zero() { return Vec{0u, 0u, 0u, 0u}; }
  static MOE_DEV Vec b_w(uint32_t w) { return magic_pairs(w); }
  static MOE_DEV Vec corr() { return Vec{kMinus136Pair, kMinus136Pair, kMinus136Pair, kMinus136Pair}; }
  static MOE_DEV f32x4_t mfma(const Vec &a, const Vec &b, const f32x4_t &c) { return mfma_bf16(a, b, c); }
};
template <>
struct MfmaFmt<MOE_W_INT8_ROW> {
  static constexpr int kBlockK = 16;
  using Vec = u32x2_t;
  static MOE_DEV Vec a_x(const uint16_t *row, int b, int g) {
    const uint2 v = reinterpret_cast<const uint2 *>(row)[4 * b + g];
    return Vec{v.x, v.y};
  }
  static MOE_DEV Vec a_plane(const uint16_t *plane, int b, int g) { return a_x(plane, b, g); }
  static MOE_DEV Vec zero() { return Vec{0u, 0u}; }
  static MOE_DEV Vec b_w(uint32_t w) { return byte_pairs(w); }
  static MOE_DEV Vec corr() { return zero(); }  // unused: q itself needs no correction
  static MOE_DEV f32x4_t mfma(const Vec &a, const Vec &b, const f32x4_t &c) { return mfma_bf16_k16(a, b, c); }
};

// A global-memory pointer that is the same in every lane, held in scalar
// registers (so that selecting between two of them per lane is a register
// select, not a load from the argument block), and typed as global so that
// the loads through it are global loads (a flat load would also count
// against the LDS counter that every LDS wait drains).
typedef __attribute__((address_space(1))) const char gchar_t;
typedef __attribute__((address_space(1))) const u32x4_t gu32x4_t;
typedef __attribute__((address_space(1))) const uint32_t gu32_t;
typedef __attribute__((address_space(1))) const u32x2_t gu2_t;
typedef __attribute__((address_space(1))) const float gf32_t;

MOE_DEV gchar_t *uniform_gptr(const void *p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<gchar_t *>((static_cast<uint64_t>(hi) << 32) | lo);
}

MOE_DEV uint4 load16_g(gchar_t *p) {
  const u32x4_t v = *reinterpret_cast<gu32x4_t *>(p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// An empty volatile statement on a 32-bit offset in registers: the
// addresses derived from it are then computed where they are used rather
// than hoisted out of the k loop and kept live (which spills, and a spill
// reload waits for every load).
MOE_DEV void pin_u32(uint32_t &v) { __asm__ volatile("" : "+v"(v)); }

template <int V>
struct IntC {
  static constexpr int value = V;
};

// step(IntC<0>), ..., step(IntC<KS - 1>) as straight-line code (k loops
// with direct loads into LDS are unrolled whole: with a loop back-edge the
// compiler waits for every outstanding load there)
template <class Fn, int... S>
MOE_DEV void unrolled_steps(std::integer_sequence<int, S...>, Fn &&step) {
  (step(IntC<S>{}), ...);
}

// s_waitcnt immediate that waits until at most n (< 64) vector memory
// requests are outstanding and leaves the other counters alone (GFX9
// encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

MOE_DEV uint4 load_stream16_g(gchar_t *p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<gu32x4_t *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

}  // namespace moe
