// Expert FFN for int4 weights on the bf16 matrix cores, decode batches.
//
// The pages stream every selected expert's weights once for all the tokens
// that picked it ("Every Public GGUF of This Model Is Missing Its Head",
// section 3; "Qwen3.6-35B-A3B: pictures, several requests at once and
// speed", Several requests at once) and fuse gate/up with the SwiGLU
// product and down with the routing weight (same page, Speed (0.1.45)).
// Here both projections are 16x16x32 bf16 MFMA tiles whose M dimension is
// the (up to 16) tokens of one expert, so the arithmetic per weight byte
// does not grow with the number of tokens sharing the expert.
//
// Exact integer operands.  A packed int4 weight q (stored as q + 8 in a
// nibble, two per byte, element 2i in the low nibble) becomes the bfloat16
// 128 + (q + 8) = q + 136 by one AND-OR (0x4300 | nibble), two nibbles per
// 32-bit word: word w gives the pairs (element s, element s + 4) for
// s = 0..3 from (w >> 4s) & 0x000F000F.  The other operand is staged in the
// same pair order.  Products of bf16 values are exact in fp32, and each
// 32-element block's sum is corrected by -136 * sum(x over the block),
// computed by one more MFMA against a constant -136 operand and fed in as
// the accumulator input, before the block's fp16 scale is applied in fp32.
// The down projection's input (the SwiGLU output, fp32) is split into
// bfloat16 hi + lo parts, which represent it to about 2^-16 relative, and
// both parts go through the matrix core.
//
// Operand layout (v_mfma_f32_16x16x32_bf16, wave64): lane l supplies A row
// l % 16 and B column l % 16, k-group l / 16 (8 consecutive k of the 32);
// the result element (m, n) lands in lane 16 * (m / 4) + n, register m % 4.
// A lane's 16-byte weight load covers one whole 32-element block of one
// row; four such loads (k-groups g = 0..3 of four consecutive blocks) are
// transposed across the four 16-lane rows of the wave with two
// permlane32 and two permlane16 swaps, after which register p of lane
// (n, g) holds k-group g of block 4j + p: exactly the B operand of that
// block's MFMA.
//
// Work split.  A block of KS waves owns one item (an expert and a tile of
// output rows); its waves split the reduction dimension and their partial
// tiles are added in LDS in wave order.  Blocks loop over items, so unused
// items cost nothing.
#include <math.h>

#include "expert_common.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr uint32_t kMagicPair = 0x43004300u;     // bf16 pair (128, 128)
constexpr uint32_t kMinus136Pair = 0xC308C308u;  // bf16 pair (-136, -136)
constexpr int kMfmaMaxWaves = 8;

MOE_DEV f32x4_t mfma_bf16(const u32x4_t &a, const u32x4_t &b, const f32x4_t &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                 c, 0, 0, 0);
}

// Eight nibbles (one k-group) -> four bf16 pairs (128 + n_s, 128 + n_{s+4}).
MOE_DEV u32x4_t magic_pairs(uint32_t w) {
  u32x4_t r;
  r.x = (w & 0x000F000Fu) | kMagicPair;
  r.y = ((w >> 4) & 0x000F000Fu) | kMagicPair;
  r.z = ((w >> 8) & 0x000F000Fu) | kMagicPair;
  r.w = ((w >> 12) & 0x000F000Fu) | kMagicPair;
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

// Position of SwiGLU column f inside its row of the act planes: the pair
// order of the MFMA operands, (f, f + 4) adjacent within each group of 8.
MOE_DEV int act_pos(int f) { return (f & ~7) | ((f & 3) << 1) | ((f >> 2) & 1); }

// Units of the MFMA kernels: the shared expert's tiles first, then the
// routed units' tiles.
struct MUnit {
  const void *gq, *gs, *uq, *us, *dq, *ds;
  int F, e, r0, n, tile;
  bool shared;
};

MOE_DEV bool mfma_unit(const FfnArgs &a, int item, int tiles_r, int tiles_s, int U, MUnit &u) {
  if (item < tiles_s) {
    u.shared = true;
    u.gq = a.sgq;
    u.gs = a.sgs;
    u.uq = a.suq;
    u.us = a.sus;
    u.dq = a.sdq;
    u.ds = a.sds;
    u.F = a.Fs;
    u.e = 0;
    u.r0 = 0;
    u.n = a.T;
    u.tile = item;
    return true;
  }
  const int i = item - tiles_s;
  const int k = i / tiles_r;
  if (k >= U) return false;
  u.shared = false;
  u.gq = a.gq;
  u.gs = a.gs;
  u.uq = a.uq;
  u.us = a.us;
  u.dq = a.dq;
  u.ds = a.ds;
  u.F = a.F;
  u.tile = i - k * tiles_r;
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

MOE_DEV int mrow_token(const FfnArgs &a, const MUnit &u, int r) {
  int t = u.shared ? r : (a.row_tok ? a.row_tok[r] : r);
  return t < 0 ? 0 : (t >= a.T ? a.T - 1 : t);  // memory safety for malformed row lists
}
MOE_DEV size_t mrow_act(const FfnArgs &a, const MUnit &u, int r) {
  return u.shared ? static_cast<size_t>(a.n_rows) * a.F + static_cast<size_t>(r) * a.Fs
                  : static_cast<size_t>(r) * a.F;
}

// ------------------------------------------------------------------ gate/up
//
// Item: (unit, 16 SwiGLU columns f0..f0+15): the 16 gate rows and the 16 up
// rows.  Wave w multiplies block-quads [w JW, w JW + JW) of the hidden
// dimension (128 elements each).  Output: act rows as bf16 hi and lo planes
// in the pair order above.
template <int JW>
__global__ void __launch_bounds__(512) gateup_mfma_kernel(FfnArgs a) {
  __shared__ f32x4_t red[kMfmaMaxWaves][2][64];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int KS = blockDim.x >> 6;
  const int n = lane & 15;
  const int g = lane >> 4;
  const int H = a.H;
  const int nsc = H / 32;
  const size_t row_bytes = static_cast<size_t>(H) / 2;
  const int U = routed_units(a);
  const int tiles_r = a.F / 16;
  const int tiles_s = a.Fs / 16;
  const int n_items = tiles_s + U * tiles_r;
  const u32x4_t m136 = {kMinus136Pair, kMinus136Pair, kMinus136Pair, kMinus136Pair};
  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};

  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    MUnit u;
    if (!mfma_unit(a, item, tiles_r, tiles_s, U, u) || u.n <= 0) continue;
    const int f0 = u.tile * 16;
    const size_t row = static_cast<size_t>(u.e) * u.F + f0 + n;
    const uint4 *gp = reinterpret_cast<const uint4 *>(static_cast<const char *>(u.gq) + row * row_bytes);
    const uint4 *up = reinterpret_cast<const uint4 *>(static_cast<const char *>(u.uq) + row * row_bytes);
    const uint32_t *gsp = reinterpret_cast<const uint32_t *>(static_cast<const uint16_t *>(u.gs) + row * nsc);
    const uint32_t *usp = reinterpret_cast<const uint32_t *>(static_cast<const uint16_t *>(u.us) + row * nsc);
    uint4 wg[JW], wu[JW];
    uint32_t sg[JW][2], su[JW][2];
#pragma unroll
    for (int jj = 0; jj < JW; ++jj) {
      const int j = wave * JW + jj;
      wg[jj] = load_stream16(gp + 4 * j + g);
      wu[jj] = load_stream16(up + 4 * j + g);
      sg[jj][0] = gsp[2 * j];
      sg[jj][1] = gsp[2 * j + 1];
      su[jj][0] = usp[2 * j];
      su[jj][1] = usp[2 * j + 1];
    }
#pragma unroll
    for (int jj = 0; jj < JW; ++jj) {
      xpose4(wg[jj]);
      xpose4(wu[jj]);
    }

    for (int m0 = 0; m0 < u.n; m0 += 16) {
      const int m = m0 + n;
      const bool mv = m < u.n;
      const uint4 *xp = reinterpret_cast<const uint4 *>(a.x + static_cast<size_t>(mrow_token(a, u, u.r0 + (mv ? m : 0))) * H);
      u32x4_t xa[JW][4];
#pragma unroll
      for (int jj = 0; jj < JW; ++jj)
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int b = 4 * (wave * JW + jj) + p;
          xa[jj][p] = pair_permute(mv ? xp[4 * b + g] : make_uint4(0, 0, 0, 0));
        }
      f32x4_t accg = zero4, accu = zero4;
#pragma unroll
      for (int jj = 0; jj < JW; ++jj)
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const f32x4_t corr = mfma_bf16(xa[jj][p], m136, zero4);
          const f32x4_t cg = mfma_bf16(xa[jj][p], magic_pairs(word(wg[jj], p)), corr);
          const f32x4_t cu = mfma_bf16(xa[jj][p], magic_pairs(word(wu[jj], p)), corr);
          accg = fma4(scale4(sg[jj][0], sg[jj][1], p), cg, accg);
          accu = fma4(scale4(su[jj][0], su[jj][1], p), cu, accu);
        }
      red[wave][0][lane] = accg;
      red[wave][1][lane] = accu;
      __syncthreads();
      if (wave == 0) {
        f32x4_t G = red[0][0][lane], V = red[0][1][lane];
        for (int w = 1; w < KS; ++w) {
          G += red[w][0][lane];
          V += red[w][1][lane];
        }
        const int f = f0 + n;
        const int pos = act_pos(f);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int mm = m0 + 4 * g + i;
          if (mm < u.n) {
            const float gv = G[i], uv = V[i];
            const float v = gv / (1.f + expf(-gv)) * uv;
            const uint16_t hi = f32_to_bf16_rne(v);
            const uint16_t lo = f32_to_bf16_rne(v - bf16_to_f32(hi));
            uint16_t *arow = reinterpret_cast<uint16_t *>(a.act + mrow_act(a, u, u.r0 + mm));
            arow[pos] = hi;
            arow[u.F + pos] = lo;
          }
        }
      }
      __syncthreads();
    }
  }
}

// --------------------------------------------------------------------- down
//
// Item: (unit, 64 output rows h0..h0+63 as four 16-row tiles).  Wave w
// multiplies block-quads [w JW, w JW + JW) of the SwiGLU dimension.  The
// routing weight is applied when the summed tile is stored.
template <int JW>
__global__ void __launch_bounds__(512) down_mfma_kernel(FfnArgs a) {
  __shared__ f32x4_t red[kMfmaMaxWaves][4][64];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int KS = blockDim.x >> 6;
  const int n = lane & 15;
  const int g = lane >> 4;
  const int H = a.H;
  const int U = routed_units(a);
  const int tiles = H / 64;
  const int n_items = (a.Fs > 0 ? tiles : 0) + U * tiles;
  const u32x4_t m136 = {kMinus136Pair, kMinus136Pair, kMinus136Pair, kMinus136Pair};
  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};

  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    MUnit u;
    if (!mfma_unit(a, item, tiles, a.Fs > 0 ? tiles : 0, U, u) || u.n <= 0) continue;
    const int h0 = u.tile * 64;
    const int F = u.F;
    const int nsc = F / 32;
    const size_t row_bytes = static_cast<size_t>(F) / 2;
    uint4 wd[JW][4];
    uint32_t sd[JW][4][2];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const size_t row = static_cast<size_t>(u.e) * H + h0 + 16 * nt + n;
      const uint4 *dp = reinterpret_cast<const uint4 *>(static_cast<const char *>(u.dq) + row * row_bytes);
      const uint32_t *sp = reinterpret_cast<const uint32_t *>(static_cast<const uint16_t *>(u.ds) + row * nsc);
#pragma unroll
      for (int jj = 0; jj < JW; ++jj) {
        const int j = wave * JW + jj;
        wd[jj][nt] = load_stream16(dp + 4 * j + g);
        sd[jj][nt][0] = sp[2 * j];
        sd[jj][nt][1] = sp[2 * j + 1];
      }
    }
#pragma unroll
    for (int jj = 0; jj < JW; ++jj)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) xpose4(wd[jj][nt]);

    for (int m0 = 0; m0 < u.n; m0 += 16) {
      const int m = m0 + n;
      const bool mv = m < u.n;
      const uint4 *hp = reinterpret_cast<const uint4 *>(a.act + mrow_act(a, u, u.r0 + (mv ? m : 0)));
      const uint4 *lp = hp + F / 8;  // lo plane follows the hi plane
      u32x4_t ah[JW][4], al[JW][4];
#pragma unroll
      for (int jj = 0; jj < JW; ++jj)
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int b = 4 * (wave * JW + jj) + p;
          const uint4 vh = mv ? hp[4 * b + g] : make_uint4(0, 0, 0, 0);
          const uint4 vl = mv ? lp[4 * b + g] : make_uint4(0, 0, 0, 0);
          ah[jj][p] = {vh.x, vh.y, vh.z, vh.w};
          al[jj][p] = {vl.x, vl.y, vl.z, vl.w};
        }
      f32x4_t acc[4] = {zero4, zero4, zero4, zero4};
#pragma unroll
      for (int jj = 0; jj < JW; ++jj)
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          f32x4_t corr = mfma_bf16(ah[jj][p], m136, zero4);
          corr = mfma_bf16(al[jj][p], m136, corr);
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) {
            const u32x4_t bw = magic_pairs(word(wd[jj][nt], p));
            f32x4_t c = mfma_bf16(ah[jj][p], bw, corr);
            c = mfma_bf16(al[jj][p], bw, c);
            acc[nt] = fma4(scale4(sd[jj][nt][0], sd[jj][nt][1], p), c, acc[nt]);
          }
        }
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) red[wave][nt][lane] = acc[nt];
      __syncthreads();
      if (wave < 4) {
        const int nt = wave;
        f32x4_t v = red[0][nt][lane];
        for (int w = 1; w < KS; ++w) v += red[w][nt][lane];
        const int h = h0 + 16 * nt + n;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int mm = m0 + 4 * g + i;
          if (mm < u.n) {
            const int r = u.r0 + mm;
            const float w = u.shared || !a.row_w ? 1.f : a.row_w[r];
            const int orow = u.shared ? a.n_rows + r : r;
            a.rows_out[static_cast<size_t>(orow) * H + h] = v[i] * w;
          }
        }
      }
      __syncthreads();
    }
  }
}

// ----------------------------------------------------------------- launches

static int mfma_grid(int items) { return items < 1 ? 1 : (items < 4096 ? items : 4096); }

template <int JW>
static hipError_t launch_gateup_mfma_t(const FfnArgs &a, int ks, hipStream_t s) {
  const int items = a.Fs / 16 + a.max_units * (a.F / 16);
  gateup_mfma_kernel<JW><<<mfma_grid(items), 64 * ks, 0, s>>>(a);
  return hipGetLastError();
}

template <int JW>
static hipError_t launch_down_mfma_t(const FfnArgs &a, int ks, hipStream_t s) {
  const int tiles = a.H / 64;
  const int items = (a.Fs > 0 ? tiles : 0) + a.max_units * tiles;
  down_mfma_kernel<JW><<<mfma_grid(items), 64 * ks, 0, s>>>(a);
  return hipGetLastError();
}

// Block-quads J = K / 128 split over KS waves of JW each, KS in {4, 8}.
static bool split_k(int K, int &jw, int &ks) {
  const int J = K / 128;
  if (K % 128 || J < 4) return false;
  ks = J <= 8 ? J : 8;
  if (ks != 4 && ks != 8) return false;
  jw = J / ks;
  return jw * ks == J && (jw == 1 || jw == 2 || jw == 4);
}

bool mfma_decode_ok(const FfnArgs &a) {
  int jw, ks;
  return a.fmt == MOE_W_INT4_B32 && a.T <= kFusedTokens && (a.Fs == 0 || a.Fs == a.F) && split_k(a.H, jw, ks) &&
         split_k(a.F, jw, ks);
}

hipError_t launch_gateup_mfma(const FfnArgs &a, hipStream_t s) {
  int jw, ks;
  split_k(a.H, jw, ks);
  if (jw == 1) return launch_gateup_mfma_t<1>(a, ks, s);
  if (jw == 2) return launch_gateup_mfma_t<2>(a, ks, s);
  return launch_gateup_mfma_t<4>(a, ks, s);
}

hipError_t launch_down_mfma(const FfnArgs &a, hipStream_t s) {
  int jw, ks;
  split_k(a.F, jw, ks);
  if (jw == 1) return launch_down_mfma_t<1>(a, ks, s);
  if (jw == 2) return launch_down_mfma_t<2>(a, ks, s);
  return launch_down_mfma_t<4>(a, ks, s);
}

}  // namespace moe
