// Expert FFN as streamed GEMVs: every selected expert's weights are read
// from HBM once, with 16-byte loads, for all the rows (tokens) that picked it
// ("Every Public GGUF of This Model Is Missing Its Head", section 3: read the
// expert weights once per row group; "Qwen3.6-35B-A3B: pictures, several
// requests at once and speed", Several requests at once: an expert shared by
// two conversations is read once for both).  Dequantisation happens in
// registers and gate/up are fused with the SwiGLU product (the pages fuse
// "gate+up+SwiGLU" into one launch, same page, Speed (0.1.45)); the down
// projection carries the routing weight.  The shared expert is one more
// unit of the same launches, so the routed and shared work of a layer is
// two launches in all (the pages' "experts eight at a time, a launch a
// stage": "Models and backends", What was tuned).
//
// Work split.  A launch walks a list of items (unit, slice); blocks loop
// over the items, so idle blocks cost nothing and the grid stays bounded.
// Inside a block each weight row belongs to a quarter-wave (16 lanes) and
// lane j of the quarter streams the row's 16-byte chunks j, j+16, ...  A
// 16-byte int4 chunk is one 32-element block with one fp16 scale.  The
// activations the rows are multiplied with are staged in LDS once per block
// (never read from global memory by every wave: thousands of waves re-reading
// the same few cache lines serialise on a handful of L2 channels), and
// results are staged in LDS so that global writes are whole row segments.
//
// int4 gate/up arithmetic.  Nibble n of a 32-bit word is turned into the
// bfloat16 128 + n with one AND-OR (0x4300 | n), two nibbles per word, and
// multiplied by bf16 activations with v_dot2c_f32_bf16.  Both operands are
// exact in bf16 and the products are exact in fp32, so the only rounding is
// the fp32 accumulation.  Since 128 + n = q + 136, each 32-element block's
// dot product is corrected by 136 * sum(x over the block) (computed once per
// token and block while the activations are staged) before its fp16 scale
// is applied in fp32.  The activations are staged pair-permuted to match the
// nibble order the AND-OR produces (elements i and i+4 of each 8-element
// word).
//
// int8 arithmetic.  q + 128 = byte ^ 0x80 is converted with v_cvt_f32_ubyte,
// accumulated in fp32 against fp32 activations, corrected by 128 * sum(x)
// per 16-element chunk, and scaled by the row's fp32 scale at the end.
//
// Down arithmetic.  Weights are dequantised to fp32 (q * s rounds once from
// the exact product) and multiplied with the fp32 SwiGLU output.
// Conversions go through unsigned values with an explicit offset: the
// toolchain folds a float conversion of a signed bit-field extract into an
// unsigned convert of the sign-extended field, which is wrong for negative
// values.
#include <math.h>

#include "expert_common.h"

namespace moe {

// ------------------------------------------------------------- gate/up

// LDS: staged activations [kGuRows][nch][XD dwords] (quads rotated by c/4
// so the 16 lanes of a quarter reading 16 consecutive chunks spread over the
// banks), per-(row, chunk) sums [kGuRows][nch], output tile [kGuRows][16]
// (8 gate values then 8 up values per row).  The 16 quarter-waves of a block
// each own one weight row: quarters 0-7 the gate rows f0..f0+7, quarters
// 8-15 the up rows.
template <int FMT, int NI>
__global__ void __launch_bounds__(256) gateup_kernel(FfnArgs a) {
  using Tr = FmtTraits<FMT>;
  constexpr int EPC = Tr::kElemsPerChunk;
  constexpr int XD = Tr::kXDwordsPerChunk;
  constexpr int QUADS = XD / 4;
  extern __shared__ uint4 smem_q[];
  const int H = a.H;
  const int nch = H / EPC;  // multiple of 16
  const int ni = nch / 16;  // <= NI
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int qg = tid >> 4;  // quarter of the block, 0..15: rows 0-7 gate, 8-15 up
  const int j = lane & 15;
  float *xsum_lds = reinterpret_cast<float *>(smem_q + static_cast<size_t>(kGuRows) * nch * QUADS);
  float *out_lds = xsum_lds + kGuRows * nch;  // [kGuRows][16]: 8 gate then 8 up values
  const size_t row_bytes = static_cast<size_t>(H) * Tr::kRowBytesPerElem2 / 2;
  (void)wave;

  const int U = routed_units(a);
  const int slices = a.F / kGuSlice;
  const int slices_sh = a.Fs / kGuSlice;
  const int n_items = U * slices + slices_sh * shared_chunks(a);
  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    Unit u;
    int slice;
    if (!item_unit(a, item, U, slices, slices_sh, u, slice) || u.n <= 0) continue;
    const int f0 = slice * kGuSlice;
    const bool is_up = qg >= kGuSlice;
    const int f = f0 + (qg & (kGuSlice - 1));
    const void *wq = is_up ? u.uq : u.gq;
    const void *wsc = is_up ? u.us : u.gs;
    const uint4 *rowp = reinterpret_cast<const uint4 *>(static_cast<const char *>(wq) +
                                                        (static_cast<size_t>(u.e) * u.F + f) * row_bytes);
    uint4 w[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i)
      if (i < ni) w[i] = load_stream16(rowp + j + 16 * i);
    float sc[NI];
    float rs = 1.f;
    if constexpr (FMT == MOE_W_INT4_B32) {
      const uint16_t *sp = static_cast<const uint16_t *>(wsc) + (static_cast<size_t>(u.e) * u.F + f) * nch;
#pragma unroll
      for (int i = 0; i < NI; ++i)
        if (i < ni) sc[i] = f16_bits_to_f32(sp[j + 16 * i]);
    } else {
      rs = static_cast<const float *>(wsc)[static_cast<size_t>(u.e) * u.F + f];
    }
    // int4: bf16 magic pairs (128 + nibble), dequantised once per item
    uint32_t wb[FMT == MOE_W_INT4_B32 ? NI : 1][16];
    if constexpr (FMT == MOE_W_INT4_B32) {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        if (i < ni) {
          const uint32_t ww[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
#pragma unroll
          for (int dd = 0; dd < 4; ++dd)
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) wb[i][4 * dd + s4] = ((ww[dd] >> (4 * s4)) & 0x000F000Fu) | 0x43004300u;
        }
      }
    }

    for (int rg = 0; rg < u.n; rg += kGuRows) {
      const int nt = min(kGuRows, u.n - rg);
      lds_barrier();  // the previous pass's LDS readers are done
      const int n_stage = nt * nch;
      for (int base = tid; base < n_stage; base += 256 * kGuStageItems) {
      uint4 raw[kGuStageItems][QUADS];
#pragma unroll
      for (int b = 0; b < kGuStageItems; ++b) {
        const int idx = base + 256 * b;
        if (idx < n_stage) {
          const int tk = idx / nch;
          const int c = idx - tk * nch;
          const int tok = unit_token(a, u, u.r0 + rg + tk);
          const uint4 *src = reinterpret_cast<const uint4 *>(a.x + static_cast<size_t>(tok) * H + c * EPC);
#pragma unroll
          for (int q = 0; q < QUADS; ++q) raw[b][q] = src[q];
        }
      }
#pragma unroll
      for (int b = 0; b < kGuStageItems; ++b) {
        const int idx = base + 256 * b;
        if (idx >= n_stage) break;
        const int tk = idx / nch;
        const int c = idx - tk * nch;
        uint32_t d[XD];
#pragma unroll
        for (int q = 0; q < QUADS; ++q) {
          const uint4 v = raw[b][q];
          d[4 * q + 0] = v.x;
          d[4 * q + 1] = v.y;
          d[4 * q + 2] = v.z;
          d[4 * q + 3] = v.w;
        }
        float s = 0.f;
#pragma unroll
        for (int m = 0; m < XD; ++m) {
          s += bf16_lo(d[m]);
          s += bf16_hi(d[m]);
        }
        uint32_t p[XD];
        if constexpr (FMT == MOE_W_INT4_B32) {
          // word g of 8 elements: pair i = (x[8g+i], x[8g+i+4]), i = 0..3
#pragma unroll
          for (int g = 0; g < 4; ++g) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const uint32_t lo = d[4 * g + i / 2], hi = d[4 * g + 2 + i / 2];
              p[4 * g + i] = (i & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
            }
          }
        } else {
#pragma unroll
          for (int m = 0; m < XD; ++m) p[m] = d[m];
        }
        uint4 *dst = smem_q + (static_cast<size_t>(tk) * nch + c) * QUADS;
#pragma unroll
        for (int q = 0; q < QUADS; ++q)
          dst[quad_slot<QUADS>(c, q)] = make_uint4(p[4 * q], p[4 * q + 1], p[4 * q + 2], p[4 * q + 3]);
        xsum_lds[tk * nch + c] = s;
      }
      }
      lds_barrier();

      for (int t = 0; t < nt; ++t) {
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          if (i >= ni) break;
          const int c = j + 16 * i;
          const uint4 *src = smem_q + (static_cast<size_t>(t) * nch + c) * QUADS;
          const float xsum = xsum_lds[t * nch + c];
          if constexpr (FMT == MOE_W_INT4_B32) {
            float d = 0.f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const uint4 v = src[quad_slot<4>(c, q)];
              d = dot2_bf16(wb[i][4 * q + 0], v.x, d);
              d = dot2_bf16(wb[i][4 * q + 1], v.y, d);
              d = dot2_bf16(wb[i][4 * q + 2], v.z, d);
              d = dot2_bf16(wb[i][4 * q + 3], v.w, d);
            }
            acc = fmaf(sc[i], fmaf(-Tr::kOffset, xsum, d), acc);
          } else {
            // q + 128 = byte ^ 0x80 as float, against the bf16 activations
            const uint32_t ww[4] = {w[i].x ^ 0x80808080u, w[i].y ^ 0x80808080u, w[i].z ^ 0x80808080u,
                                    w[i].w ^ 0x80808080u};
            float d = 0.f;
#pragma unroll
            for (int q = 0; q < 2; ++q) {
              const uint4 v = src[quad_slot<2>(c, q)];
              const uint32_t xv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
              for (int m = 0; m < 4; ++m) {
                // x dword m of quad q holds elements 8q + 2m and 8q + 2m + 1
                const uint32_t wd = ww[2 * q + m / 2];
                const float w0 = (m & 1) ? ubyte_f32<2>(wd) : ubyte_f32<0>(wd);
                const float w1 = (m & 1) ? ubyte_f32<3>(wd) : ubyte_f32<1>(wd);
                d = fmaf(w0, bf16_lo(xv[m]), d);
                d = fmaf(w1, bf16_hi(xv[m]), d);
              }
            }
            acc += fmaf(-Tr::kOffset, xsum, d);
          }
        }
        const float r = sum16(acc) * rs;
        if (j == 0) out_lds[t * 16 + qg] = r;
      }
      lds_barrier();
      if (tid < nt * kGuSlice) {
        const int t = tid / kGuSlice, fl = tid - t * kGuSlice;
        const float g = out_lds[t * 16 + fl];
        const float uu = out_lds[t * 16 + kGuSlice + fl];
        a.act[unit_act_off(a, u, u.r0 + rg + t) + f0 + fl] = g / (1.f + expf(-g)) * uu;
      }
    }
  }
}

// ------------------------------------------------------------- down

// LDS: staged SwiGLU rows [kDnRows][F] fp32 (the eight 16-byte groups of
// each 128-byte chunk rotated by the chunk index), output tile
// [kDnRows][kDnSlice].

template <int FMT, int NI>
__global__ void __launch_bounds__(256) down_kernel(FfnArgs a) {
  using Tr = FmtTraits<FMT>;
  constexpr int EPC = Tr::kElemsPerChunk;  // 32 (int4) or 16 (int8) weights per 16 bytes
  extern __shared__ float4 smem_f4[];
  const int H = a.H;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int quarter = lane >> 4;
  const int j = lane & 15;

  const int U = routed_units(a);
  const int slices = H / kDnSlice;
  const int n_items = U * slices + slices * shared_chunks(a);
  const int fmax = a.F > a.Fs ? a.F : a.Fs;
  float *out_lds = reinterpret_cast<float *>(smem_f4 + static_cast<size_t>(kDnRows) * (fmax / 4));
  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    Unit u;
    int slice;
    if (!item_unit(a, item, U, slices, slices, u, slice) || u.n <= 0) continue;
    const int F = u.F;
    const int nch = F / EPC;  // multiple of 16
    const int ni = nch / 16;  // <= NI
    const int f4 = F / 4;     // float4 per act row
    const int h0 = slice * kDnSlice;
    const size_t row_bytes = static_cast<size_t>(F) * Tr::kRowBytesPerElem2 / 2;
    // this wave's 4 row-quads: rows h0 + 16*wave + 4*rq + quarter
    uint4 wd[4][NI];
    float sd[4][NI];
    float rsc[4];
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int h = h0 + 16 * wave + 4 * rq + quarter;
      const uint4 *dq = reinterpret_cast<const uint4 *>(static_cast<const char *>(u.dq) +
                                                        (static_cast<size_t>(u.e) * H + h) * row_bytes);
#pragma unroll
      for (int i = 0; i < NI; ++i) wd[rq][i] = i < ni ? load_stream16(dq + j + 16 * i) : make_uint4(0, 0, 0, 0);
      if constexpr (FMT == MOE_W_INT4_B32) {
        const uint16_t *ds = static_cast<const uint16_t *>(u.ds) + (static_cast<size_t>(u.e) * H + h) * nch;
#pragma unroll
        for (int i = 0; i < NI; ++i) sd[rq][i] = i < ni ? f16_bits_to_f32(ds[j + 16 * i]) : 0.f;
        rsc[rq] = 1.f;
      } else {
        rsc[rq] = static_cast<const float *>(u.ds)[static_cast<size_t>(u.e) * H + h];
#pragma unroll
        for (int i = 0; i < NI; ++i) sd[rq][i] = 1.f;
      }
    }

    for (int rg = 0; rg < u.n; rg += kDnRows) {
      const int nt = min(kDnRows, u.n - rg);
      lds_barrier();
      // batches of independent 16-byte loads, then their LDS stores
      const int n4 = nt * f4;
      for (int base = tid; base < n4; base += 256 * kStageBatch) {
        float4 v[kStageBatch];
#pragma unroll
        for (int b = 0; b < kStageBatch; ++b) {
          const int idx = base + 256 * b;
          const int t = idx / f4;
          const int k4 = idx - t * f4;
          v[b] = idx < n4 ? reinterpret_cast<const float4 *>(a.act + unit_act_off(a, u, u.r0 + rg + t))[k4]
                          : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int b = 0; b < kStageBatch; ++b) {
          const int idx = base + 256 * b;
          if (idx < n4) {
            const int t = idx / f4;
            const int k4 = idx - t * f4;
            smem_f4[static_cast<size_t>(t) * f4 + act_slot(k4 >> 3, k4 & 7)] = v[b];
          }
        }
      }
      lds_barrier();
      // one row at a time (runtime loop keeps a single fp32 fragment live;
      // the selection below costs a few scratch accesses per row)
#pragma unroll 1
      for (int rq = 0; rq < 4; ++rq) {
        uint4 wr[NI];
        float sr[NI];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          wr[i] = rq == 0 ? wd[0][i] : rq == 1 ? wd[1][i] : rq == 2 ? wd[2][i] : wd[3][i];
          sr[i] = rq == 0 ? sd[0][i] : rq == 1 ? sd[1][i] : rq == 2 ? sd[2][i] : sd[3][i];
        }
        const float rr = rq == 0 ? rsc[0] : rq == 1 ? rsc[1] : rq == 2 ? rsc[2] : rsc[3];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          if (i >= ni) break;
          float wf[EPC];
          const uint32_t w4[4] = {wr[i].x, wr[i].y, wr[i].z, wr[i].w};
          if constexpr (FMT == MOE_W_INT4_B32) {
            // element 8*dd + n is nibble n of word dd, stored as q + 8
            const float off = -8.f * sr[i];
#pragma unroll
            for (int dd = 0; dd < 4; ++dd)
#pragma unroll
              for (int n = 0; n < 8; ++n)
                wf[8 * dd + n] = fmaf(static_cast<float>((w4[dd] >> (4 * n)) & 0xFu), sr[i], off);
          } else {
#pragma unroll
            for (int dd = 0; dd < 4; ++dd) {
              const uint32_t v = w4[dd] ^ 0x80808080u;  // byte ^ 0x80 = q + 128
              wf[4 * dd + 0] = ubyte_f32<0>(v) - 128.f;
              wf[4 * dd + 1] = ubyte_f32<1>(v) - 128.f;
              wf[4 * dd + 2] = ubyte_f32<2>(v) - 128.f;
              wf[4 * dd + 3] = ubyte_f32<3>(v) - 128.f;
            }
          }
          // chunk c of the row covers act floats [c*EPC, c*EPC + EPC)
          const int c = j + 16 * i;
          for (int t = 0; t < nt; ++t) {
            const float4 *row = smem_f4 + static_cast<size_t>(t) * f4;
            float d = 0.f;
#pragma unroll
            for (int q = 0; q < EPC / 4; ++q) {
              const int k4 = c * (EPC / 4) + q;  // float4 index in the row
              const float4 v = row[act_slot(k4 >> 3, k4 & 7)];
              d = fmaf(wf[4 * q], v.x, d);
              d = fmaf(wf[4 * q + 1], v.y, d);
              d = fmaf(wf[4 * q + 2], v.z, d);
              d = fmaf(wf[4 * q + 3], v.w, d);
            }
            d = sum16(d) * rr;
            if (j == 0) {
              float *o = out_lds + t * kDnSlice + 16 * wave + 4 * rq + quarter;
              *o = (i == 0) ? d : *o + d;
            }
          }
        }
      }
      lds_barrier();
      {  // one float4 of the [nt][64] tile per thread, scaled by the row weight
        const int t = tid >> 4, h4 = tid & 15;
        if (t < nt) {
          const int r = u.r0 + rg + t;
          const float w = unit_row_w(a, u, r);
          float4 v = reinterpret_cast<const float4 *>(out_lds + t * kDnSlice)[h4];
          v.x *= w;
          v.y *= w;
          v.z *= w;
          v.w *= w;
          reinterpret_cast<float4 *>(a.rows_out + static_cast<size_t>(unit_out_row(a, u, r)) * H + h0)[h4] = v;
        }
      }
    }
  }
}

// ------------------------------------------------------------- launches

template <int FMT>
static size_t gateup_lds_bytes(int H) {
  using Tr = FmtTraits<FMT>;
  const int nch = H / Tr::kElemsPerChunk;
  return static_cast<size_t>(kGuRows) * nch * (Tr::kXDwordsPerChunk * 4 + 4) + kGuRows * 16 * 4;
}

static size_t down_lds_bytes(int F, int Fs) {
  const int fmax = F > Fs ? F : Fs;
  return static_cast<size_t>(kDnRows) * fmax * 4 + kDnRows * kDnSlice * 4;
}

static int grid_for(int items) { return items < 1 ? 1 : (items < 2048 ? items : 2048); }

template <typename K>
static hipError_t set_lds(K kernel, size_t lds) {
  if (lds <= 64 * 1024) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void *>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                             static_cast<int>(lds));
}

static int max_items(const FfnArgs &a, int slices, int slices_sh) {
  const int chunks = a.Fs > 0 ? (a.T + kSharedChunk - 1) / kSharedChunk : 0;
  return a.max_units * slices + slices_sh * chunks;
}

template <int FMT, int NI>
static hipError_t launch_gateup_t(const FfnArgs &a, hipStream_t s) {
  const size_t lds = gateup_lds_bytes<FMT>(a.H);
  hipError_t e = set_lds(gateup_kernel<FMT, NI>, lds);
  if (e != hipSuccess) return e;
  const int items = max_items(a, a.F / kGuSlice, a.Fs / kGuSlice);
  return launch_kernel(gateup_kernel<FMT, NI>, dim3(grid_for(items)), dim3(256), lds, s, a.ev, a);
}

template <int FMT, int NI>
static hipError_t launch_down_t(const FfnArgs &a, hipStream_t s) {
  const size_t lds = down_lds_bytes(a.F, a.Fs);
  hipError_t e = set_lds(down_kernel<FMT, NI>, lds);
  if (e != hipSuccess) return e;
  const int items = max_items(a, a.H / kDnSlice, a.H / kDnSlice);
  return launch_kernel(down_kernel<FMT, NI>, dim3(grid_for(items)), dim3(256), lds, s, a.ev, a);
}

template <int FMT>
static hipError_t launch_gateup_fmt(const FfnArgs &a, hipStream_t s) {
  constexpr int EPC = FmtTraits<FMT>::kElemsPerChunk;
  const int ni = a.H / EPC / 16;
  if (ni <= 1) return launch_gateup_t<FMT, 1>(a, s);
  if (ni <= 2) return launch_gateup_t<FMT, 2>(a, s);
  if (ni <= 4) return launch_gateup_t<FMT, 4>(a, s);
  return launch_gateup_t<FMT, 8>(a, s);
}

template <int FMT>
static hipError_t launch_down_fmt(const FfnArgs &a, hipStream_t s) {
  constexpr int EPC = FmtTraits<FMT>::kElemsPerChunk;
  const int fmax = a.F > a.Fs ? a.F : a.Fs;
  const int ni = fmax / EPC / 16;
  if (ni <= 1) return launch_down_t<FMT, 1>(a, s);
  if (ni <= 2) return launch_down_t<FMT, 2>(a, s);
  return launch_down_t<FMT, 4>(a, s);
}

hipError_t launch_gateup_items(const FfnArgs &a, hipStream_t s) {
  if (a.fmt == MOE_W_INT4_B32) return launch_gateup_fmt<MOE_W_INT4_B32>(a, s);
  return launch_gateup_fmt<MOE_W_INT8_ROW>(a, s);
}

hipError_t launch_down_items(const FfnArgs &a, hipStream_t s) {
  if (a.fmt == MOE_W_INT4_B32) return launch_down_fmt<MOE_W_INT4_B32>(a, s);
  return launch_down_fmt<MOE_W_INT8_ROW>(a, s);
}

// Gate/up and down always take the same family (the SwiGLU rows' format
// differs between them).
hipError_t launch_gateup(const FfnArgs &a, hipStream_t s) {
  if (mfma_decode_ok(a)) return launch_gateup_mfma(a, s);
  if (prefill_ok(a)) return launch_gateup_prefill(a, s);
  return launch_gateup_items(a, s);
}
hipError_t launch_down(const FfnArgs &a, hipStream_t s) {
  if (mfma_decode_ok(a)) return launch_down_mfma(a, s);
  if (prefill_ok(a)) return launch_down_prefill(a, s);
  return launch_down_items(a, s);
}

}  // namespace moe
