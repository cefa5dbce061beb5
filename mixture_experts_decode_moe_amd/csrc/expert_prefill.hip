// Expert FFN for large batches (prefill chunks), int4 weights: grouped
// GEMMs on the bf16 matrix cores.
//
// Which path runs depends on how many rows each expert serves; the pages
// measure the crossover from per-row kernels to a dense contraction in rows
// per expert ("Strata on an Intel Arc", prompt processing).  A prefill chunk
// gives every expert tens of rows (2048 tokens x 8 slots over 256 experts is
// 64 on average), enough to tile each expert's rows as the M dimension of a
// GEMM and reuse every weight tile across them.
//
// Two sets of kernels: pipelined GEMMs for the layer's shape (H = 2048,
// F = 512; further below) and generic ones for any other shape.  The
// generic kernels compute as the decode kernels do (expert_mfma.hip): the int4 weights
// enter the MFMA as the exact bfloat16 values 128 + nibble = q + 136, the
// other operand is exact (x in bf16; the SwiGLU output as bf16 hi + lo), the
// fp32 accumulator input of each 32-element block is -136 * sum(other
// operand over the block) (computed while the operand tile is staged), and
// the block's fp16 scale is applied with an fp32 FMA.
//
// Generic tiles.  An item is (unit, 64 rows, 64 output columns); a block of 4 waves
// works on it, wave w owning the 16 columns 16w..16w+15 of all 64 rows (four
// 16x16 MFMA tiles along M).  Gate/up items hold 64 SwiGLU columns, i.e. 64
// gate and the matching 64 up columns, so wave w has both halves of its
// SwiGLU columns in registers.  The reduction dimension advances in steps
// of 128 (four 32-element blocks): the A tile (the unit's rows, gathered
// for gate/up) is double-buffered in LDS with its block sums, the weight
// chunks of the next step are loaded into registers while the current step
// is multiplied.  Blocks loop over the items; units and their row tiles are
// enumerated once per block into an LDS table.
#include <math.h>

#include "mfma_common.h"

namespace moe {

constexpr int kPfRows = 64;      // rows per item
constexpr int kPfCols = 64;      // output columns per item (gate/up: SwiGLU columns)
constexpr int kPfMaxUnits = 1040;  // shared expert + up to 1024 routed + slack
constexpr int kPfThreads = 256;

// Unit u of the call: the shared expert first (when present), then the
// routed active experts in order.
struct PfUnit {
  int e;   // expert index (-1: shared)
  int r0;  // first row
  int n;   // rows
};

MOE_DEV PfUnit pf_unit(const FfnArgs &a, int u) {
  PfUnit x;
  if (a.Fs > 0) {
    if (u == 0) {
      x.e = -1;
      x.r0 = 0;
      x.n = a.T;
      return x;
    }
    --u;
  }
  if (a.offsets) {
    x.e = a.active[u];
    x.r0 = a.offsets[x.e];
    x.n = a.offsets[x.e + 1] - x.r0;
  } else {
    x.e = 0;
    x.r0 = 0;
    x.n = a.n_rows;
  }
  return x;
}

// Fills pre[u] = first row tile of unit u (exclusive prefix of the row
// tiles), pre[n_units] = total; returns the number of units.
// NT threads (scratch holds NT / 64 ints).
template <int NT = kPfThreads, int ROWS = kPfRows>
MOE_DEV int pf_tiles(const FfnArgs &a, int *pre, int *scratch) {
  const int n_units = (a.Fs > 0 ? 1 : 0) + routed_units(a);
  const int tid = threadIdx.x;
  constexpr int kPer = (kPfMaxUnits + NT - 1) / NT;
  int cnt[kPer];
  int mine = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int u = tid * kPer + i;
    int c = 0;
    if (u < n_units) {
      const PfUnit x = pf_unit(a, u);
      c = x.n > 0 ? (x.n + ROWS - 1) / ROWS : 0;
    }
    cnt[i] = c;
    mine += c;
  }
  // block exclusive scan of the per-thread totals
  const int lane = tid & 63, wave = tid >> 6;
  int inc = mine;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(inc, off);
    if (lane >= off) inc += o;
  }
  if (lane == 63) scratch[wave] = inc;
  lds_barrier();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += scratch[w];
  base += inc - mine;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int u = tid * kPer + i;
    if (u <= n_units) pre[u] = base;
    base += cnt[i];
  }
  lds_barrier();
  return n_units;
}

// Unit of row tile j (binary search in the prefix table).
MOE_DEV int pf_find(const int *pre, int n_units, int j) {
  int lo = 0, hi = n_units - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pre[mid] <= j)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

// LDS tile of the A operand: 64 rows x one k-step, 16-byte pieces (8 bf16 in
// operand order), rows padded by one piece; plus -136 * block sums [4][64].
template <int PLANES>
struct PfTile {
  uint4 a[PLANES][kPfRows][17];
  float corr[4][kPfRows];
};

// ------------------------------------------------------------------ gate/up

__global__ void __launch_bounds__(kPfThreads) gateup_prefill_kernel(FfnArgs a) {
  __shared__ PfTile<1> tile[2];
  __shared__ int pre[kPfMaxUnits + 1];
  __shared__ int scratch[4];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int n = lane & 15, g = lane >> 4;
  const int H = a.H, T = a.T;
  const int n_units = pf_tiles(a, pre, scratch);
  const int col_groups = a.F / kPfCols;  // the shared expert has Fs == F on this path
  const int n_items = pre[n_units] * col_groups;
  const int steps = H / 128;
  const int nblk = H / 32;
  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};

  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int j = item / col_groups;
    const int cg = item - j * col_groups;
    const int u = pf_find(pre, n_units, j);
    const PfUnit un = pf_unit(a, u);
    const int m0 = (j - pre[u]) * kPfRows;  // first row of the tile inside the unit
    const int rows = min(kPfRows, un.n - m0);
    const bool shared = un.e < 0;
    const int F = shared ? a.Fs : a.F;
    const int f = cg * kPfCols + 16 * wave + n;  // this lane's SwiGLU column
    const size_t wrow = static_cast<size_t>(shared ? 0 : un.e) * F + f;
    gchar_t *gq = uniform_gptr(shared ? a.sgq : a.gq) + wrow * nblk * 16;
    gchar_t *uq = uniform_gptr(shared ? a.suq : a.uq) + wrow * nblk * 16;
    gu32_t *gs = reinterpret_cast<gu32_t *>(uniform_gptr(shared ? a.sgs : a.gs) + wrow * nblk * 2);
    gu32_t *us = reinterpret_cast<gu32_t *>(uniform_gptr(shared ? a.sus : a.us) + wrow * nblk * 2);

    // A staging: thread t owns pieces t + 256 i (i < 4): row p / 16, piece p % 16
    int tok[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (tid >> 4) + 16 * i;
      int t = 0;
      if (r < rows) {
        const int rr = un.r0 + m0 + r;
        t = shared ? rr : (a.row_tok ? a.row_tok[rr] : rr);
        t = t < 0 ? 0 : (t >= T ? T - 1 : t);
      }
      tok[i] = t;
    }
    const int pc = tid & 15;
    auto load_a = [&](int s, uint4 (&v)[4]) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = (tid >> 4) + 16 * i;
        v[i] = r < rows ? reinterpret_cast<const uint4 *>(a.x + static_cast<size_t>(tok[i]) * H)[16 * s + pc]
                        : make_uint4(0, 0, 0, 0);
      }
    };
    auto store_a = [&](int buf, const uint4 (&v)[4]) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = (tid >> 4) + 16 * i;
        const u32x4_t pp = pair_permute(v[i]);
        tile[buf].a[0][r][pc] = make_uint4(pp.x, pp.y, pp.z, pp.w);
        float sum = 0.f;
        const uint32_t d[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) sum += bf16_lo(d[q]) + bf16_hi(d[q]);
        // four consecutive lanes hold one 32-element block of the row
        sum += dpp_f32<0xB1>(sum);
        sum += dpp_f32<0x4E>(sum);
        if ((pc & 3) == 0) tile[buf].corr[pc >> 2][r] = -136.f * sum;
      }
    };
    auto load_b = [&](int s, uint4 &wg, uint4 &wu, uint32_t (&sg)[2], uint32_t (&su)[2]) {
      wg = load_stream16_g(gq + 16 * (4 * s + g));
      wu = load_stream16_g(uq + 16 * (4 * s + g));
      sg[0] = gs[2 * s];
      sg[1] = gs[2 * s + 1];
      su[0] = us[2 * s];
      su[1] = us[2 * s + 1];
    };

    f32x4_t accg[4], accu[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) accg[mt] = accu[mt] = zero4;
    uint4 av[4];
    uint4 wg, wu;
    uint32_t sg[2], su[2];
    load_a(0, av);
    load_b(0, wg, wu, sg, su);
    store_a(0, av);
    lds_barrier();
    for (int s = 0; s < steps; ++s) {
      const int buf = s & 1;
      uint4 nwg, nwu;
      uint32_t nsg[2], nsu[2];
      const bool more = s + 1 < steps;
      if (more) {
        load_a(s + 1, av);
        load_b(s + 1, nwg, nwu, nsg, nsu);
      }
      xpose4(wg);
      xpose4(wu);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const u32x4_t bg = magic_pairs(word(wg, p));
        const u32x4_t bu = magic_pairs(word(wu, p));
        const float scg = scale4(sg[0], sg[1], p), scu = scale4(su[0], su[1], p);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const uint4 av4 = tile[buf].a[0][16 * mt + n][4 * p + g];
          const u32x4_t A = {av4.x, av4.y, av4.z, av4.w};
          const float4 c4 = *reinterpret_cast<const float4 *>(&tile[buf].corr[p][16 * mt + 4 * g]);
          const f32x4_t C = {c4.x, c4.y, c4.z, c4.w};
          accg[mt] = fma4(scg, mfma_bf16(A, bg, C), accg[mt]);
          accu[mt] = fma4(scu, mfma_bf16(A, bu, C), accu[mt]);
        }
      }
      if (more) {
        store_a(buf ^ 1, av);
        wg = nwg;
        wu = nwu;
        sg[0] = nsg[0];
        sg[1] = nsg[1];
        su[0] = nsu[0];
        su[1] = nsu[1];
      }
      lds_barrier();
    }
    // SwiGLU; lane (n, g) holds rows 16 mt + 4 g + i of column f
    const int pos = act_pos<MOE_W_INT4_B32>(f);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * mt + 4 * g + i;
        if (r < rows) {
          const float gv = accg[mt][i], uv = accu[mt][i];
          const float v = gv / (1.f + expf(-gv)) * uv;
          const uint16_t hi = f32_to_bf16_rne(v);
          const uint16_t lo = f32_to_bf16_rne(v - bf16_to_f32(hi));
          const int rr = m0 + r;
          const size_t off = shared ? static_cast<size_t>(a.n_rows) * a.F + static_cast<size_t>(rr) * a.Fs
                                    : static_cast<size_t>(un.r0 + rr) * a.F;
          uint16_t *arow = reinterpret_cast<uint16_t *>(a.act + off);
          arow[pos] = hi;
          arow[F + pos] = lo;
        }
      }
  }
}

// --------------------------------------------------------------------- down

__global__ void __launch_bounds__(kPfThreads) down_prefill_kernel(FfnArgs a) {
  __shared__ PfTile<2> tile[2];
  __shared__ int pre[kPfMaxUnits + 1];
  __shared__ int scratch[4];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int n = lane & 15, g = lane >> 4;
  const int H = a.H;
  const int n_units = pf_tiles(a, pre, scratch);
  const int col_groups = H / kPfCols;
  const int n_items = pre[n_units] * col_groups;
  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};

  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int j = item / col_groups;
    const int cg = item - j * col_groups;
    const int u = pf_find(pre, n_units, j);
    const PfUnit un = pf_unit(a, u);
    const int m0 = (j - pre[u]) * kPfRows;
    const int rows = min(kPfRows, un.n - m0);
    const bool shared = un.e < 0;
    const int F = shared ? a.Fs : a.F;
    const int steps = F / 128;
    const int nblk = F / 32;
    const int h = cg * kPfCols + 16 * wave + n;  // this lane's output column
    const size_t wrow = static_cast<size_t>(shared ? 0 : un.e) * H + h;
    gchar_t *dq = uniform_gptr(shared ? a.sdq : a.dq) + wrow * nblk * 16;
    gu32_t *ds = reinterpret_cast<gu32_t *>(uniform_gptr(shared ? a.sds : a.ds) + wrow * nblk * 2);

    // A staging: thread t owns pieces t + 256 i (i < 4) of both planes
    const int pc = tid & 15;
    auto arow = [&](int r) -> const uint4 * {
      const int rr = m0 + r;
      const size_t off = shared ? static_cast<size_t>(a.n_rows) * a.F + static_cast<size_t>(rr) * a.Fs
                                : static_cast<size_t>(un.r0 + rr) * a.F;
      return reinterpret_cast<const uint4 *>(a.act + off);
    };
    auto load_a = [&](int s, uint4 (&vh)[4], uint4 (&vl)[4]) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = (tid >> 4) + 16 * i;
        const uint4 *p = arow(r < rows ? r : 0);
        vh[i] = r < rows ? p[16 * s + pc] : make_uint4(0, 0, 0, 0);
        vl[i] = r < rows ? p[F / 8 + 16 * s + pc] : make_uint4(0, 0, 0, 0);
      }
    };
    auto store_a = [&](int buf, const uint4 (&vh)[4], const uint4 (&vl)[4]) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = (tid >> 4) + 16 * i;
        tile[buf].a[0][r][pc] = vh[i];
        tile[buf].a[1][r][pc] = vl[i];
        float sum = 0.f;
        const uint32_t d[8] = {vh[i].x, vh[i].y, vh[i].z, vh[i].w, vl[i].x, vl[i].y, vl[i].z, vl[i].w};
#pragma unroll
        for (int q = 0; q < 8; ++q) sum += bf16_lo(d[q]) + bf16_hi(d[q]);
        sum += dpp_f32<0xB1>(sum);
        sum += dpp_f32<0x4E>(sum);
        if ((pc & 3) == 0) tile[buf].corr[pc >> 2][r] = -136.f * sum;
      }
    };
    auto load_b = [&](int s, uint4 &w, uint32_t (&sc)[2]) {
      w = load_stream16_g(dq + 16 * (4 * s + g));
      sc[0] = ds[2 * s];
      sc[1] = ds[2 * s + 1];
    };

    f32x4_t acc[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) acc[mt] = zero4;
    uint4 vh[4], vl[4];
    uint4 w;
    uint32_t sc[2];
    load_a(0, vh, vl);
    load_b(0, w, sc);
    store_a(0, vh, vl);
    lds_barrier();
    for (int s = 0; s < steps; ++s) {
      const int buf = s & 1;
      uint4 nw;
      uint32_t nsc[2];
      const bool more = s + 1 < steps;
      if (more) {
        load_a(s + 1, vh, vl);
        load_b(s + 1, nw, nsc);
      }
      xpose4(w);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const u32x4_t b = magic_pairs(word(w, p));
        const float scp = scale4(sc[0], sc[1], p);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const uint4 h4 = tile[buf].a[0][16 * mt + n][4 * p + g];
          const uint4 l4 = tile[buf].a[1][16 * mt + n][4 * p + g];
          const u32x4_t Ah = {h4.x, h4.y, h4.z, h4.w}, Al = {l4.x, l4.y, l4.z, l4.w};
          const float4 c4 = *reinterpret_cast<const float4 *>(&tile[buf].corr[p][16 * mt + 4 * g]);
          const f32x4_t C = {c4.x, c4.y, c4.z, c4.w};
          f32x4_t c = mfma_bf16(Ah, b, C);
          c = mfma_bf16(Al, b, c);
          acc[mt] = fma4(scp, c, acc[mt]);
        }
      }
      if (more) {
        store_a(buf ^ 1, vh, vl);
        w = nw;
        sc[0] = nsc[0];
        sc[1] = nsc[1];
      }
      lds_barrier();
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * mt + 4 * g + i;
        if (r < rows) {
          const int rr = m0 + r;
          const int row = un.r0 + rr;
          const float wgt = shared || !a.row_w ? 1.f : a.row_w[row];
          const size_t orow = shared ? static_cast<size_t>(a.n_rows) + rr : static_cast<size_t>(row);
          a.rows_out[orow * H + h] = acc[mt][i] * wgt;
        }
      }
  }
}

// ------------------------------------------------ pipelined GEMM variants
// The k loop runs over groups of steps whose register slots and LDS buffers
// have constant indices, with no copies between iterations (a register ring
// copied across a loop back-edge makes the compiler wait for every load).
// Down (F = 512: four steps) stages both operands of the next step in LDS,
// two blocks per compute unit.  Gate/up
// (H = 2048: sixteen steps) runs one block per compute unit with 256
// registers a lane and keeps the weights of the next four steps and the A
// rows of the next two in flight.  Items are 64 rows by 128 SwiGLU columns
// (gate/up) or 256 output columns (down); each wave owns one 32-column
// weight tile against the 32-row tiles of A, on the 32x32x16 fp16 matrix
// instruction (measured on this chip: about 2.1 PFLOP/s against 1.2-1.3 for
// the 16x16x32 shape).  A gate/up wave's 32 columns are the gate and up
// rows of 16 SwiGLU columns, paired across lanes in the epilogue.
//
// Unlike the generic kernels, these multiply in fp16: each weight is
// dequantized once per item to the fp16 value q s (rounded once, relative
// error at most 2^-11), the x rows are staged in fp16 (bf16 values, exact
// in fp16 within its normal range), and the SwiGLU rows are handed from
// gate/up to down rounded once to fp16 (one plane), so the products
// accumulate in the matrix core with no sum correction and no per-block
// scaling on the vector unit.  Measured against the oracle: 3.6e-4 to
// 4.3e-4 of max|ref| on prefill calls (T = 37 to 2048).  The int4
// dequantization costs about 15 vector operations per 8 weights, as much
// vector time as the 32x32 tiles' matrix time at 64 rows per item; the
// 128-row gate/up items halve its share.
//
// The k loop is instantiated once per number of 32-row tiles that hold rows
// (1, 2), chosen per item: no matrix-core instruction sits under a branch.
// (With the tile count as a branch inside the loop, hipcc left an MFMA
// result read by a VALU instruction right after the branch without the
// wait states the matrix core needs, and those reads saw stale registers.)



template <class Fn>
MOE_DEV void with_msub(int msub, Fn &&fn) {
  switch (msub) {
    case 1:
      fn(IntC<1>{});
      break;
    case 2:
      fn(IntC<2>{});
      break;
    case 3:
      fn(IntC<3>{});
      break;
    default:
      fn(IntC<4>{});
      break;
  }
}

template <class Fn>
MOE_DEV void with_msub2(int msub, Fn &&fn) {
  if (msub <= 1)
    fn(IntC<1>{});
  else
    fn(IntC<2>{});
}


// 32x32 output tiles (v_mfma_f32_32x32x16_f16, twice the rate of the 16x16
// shape on this chip): lane l holds row l % 32 of A and column l % 32 of B
// with k-group l / 32 (8 consecutive k, pair-permuted) of each 16-k step,
// and accumulator j of column l % 32, row (j & 3) + 8 (j >> 2) + 4 (l / 32).
typedef float f32x16_t __attribute__((ext_vector_type(16)));

MOE_DEV f32x16_t zero16() {
  f32x16_t z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

MOE_DEV f32x16_t mfma32_f16(const u32x4_t &a, const u32x4_t &b, const f32x16_t &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                0, 0, 0);
}

// A 16-byte weight chunk (one 32-element block, its four k-group words)
// per lane, block b0 in lanes 0-31 and block b1 in lanes 32-63 (same
// column) -> lane half h holds words h and 2 + h of b0, then of b1: the
// k-groups it multiplies in the two 16-k steps of each block.
MOE_DEV void half_exchange(uint4 &v) {
  const auto a = __builtin_amdgcn_permlane32_swap(v.x, v.y, false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(v.z, v.w, false, false);
  v = make_uint4(a[0], b[0], a[1], b[1]);
}

constexpr int kGmThreads = 512;  // 8 waves; two blocks per compute unit
constexpr int kGmMaxUnits = 257;  // the shared expert and up to 256 routed experts

// The call's units in LDS, filled once per block: pre[u] = first row tile of
// unit u (pre[n] = the total), and each unit's expert (-1: shared), first
// row and row count, so that an item needs no global lookup before its
// weight requests.
struct GmUnits {
  int pre[kGmMaxUnits + 1];
  int e[kGmMaxUnits], r0[kGmMaxUnits], n[kGmMaxUnits];
};

template <int ROWS = kPfRows>
MOE_DEV int gm_units(const FfnArgs &a, GmUnits &G, int *scratch) {
  static_assert(kGmThreads >= kGmMaxUnits, "one unit per thread");
  const int n_units = (a.Fs > 0 ? 1 : 0) + routed_units(a);
  const int tid = threadIdx.x;
  int c = 0;
  if (tid < n_units) {
    const PfUnit x = pf_unit(a, tid);
    G.e[tid] = x.e;
    G.r0[tid] = x.r0;
    G.n[tid] = x.n;
    c = x.n > 0 ? (x.n + ROWS - 1) / ROWS : 0;
  }
  const int lane = tid & 63, wave = tid >> 6;
  int inc = c;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(inc, off);
    if (lane >= off) inc += o;
  }
  if (lane == 63) scratch[wave] = inc;
  lds_barrier();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += scratch[w];
  base += inc - c;
  if (tid <= n_units) G.pre[tid] = base;
  lds_barrier();
  return n_units;
}

MOE_DEV PfUnit gm_unit(const GmUnits &G, int u) {
  PfUnit x;
  x.e = G.e[u];
  x.r0 = G.r0[u];
  x.n = G.n[u];
  return x;
}

template <int KS>
__global__ void __launch_bounds__(kGmThreads, 2) gateup_gemm_kernel(FfnArgs a) {
  static_assert(KS % 4 == 0, "the k loop runs over groups of four steps");
  __shared__ uint4 as[2][kPfRows][17];  // x rows of the tile, pair-permuted fp16, one k-step
  __shared__ GmUnits units;
  __shared__ int scratch[kGmThreads / 64];
  constexpr int nblk = 4 * KS;  // 32-element blocks per weight row
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int c = lane & 31, h = lane >> 5;
  const bool up_lane = c >= 16;
  const int T = a.T;
  const int H = 128 * KS;
  const int n_units = gm_units(a, units, scratch);
  const int col_tiles = a.F / 128;
  const int n_items = units.pre[n_units] * col_tiles;
  const int pc = tid & 15;

  // XCD-aware order: the blocks of one XCD (block b runs on XCD b mod 8)
  // take a contiguous run of items per round, so the column tiles of a row
  // tile, and consecutive row tiles of a unit, share that XCD's L2 for
  // their A rows and weights
  const int per_xcd = gridDim.x >> 3;
  const int my_off = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  for (int round = 0; round < n_items; round += gridDim.x) {
    const int item = round + my_off;
    if (item >= n_items) continue;
    const int j = item / col_tiles;
    const int ct = item - j * col_tiles;
    const int u = pf_find(units.pre, n_units, j);
    const PfUnit un = gm_unit(units, u);
    const int m0 = (j - units.pre[u]) * kPfRows;
    const int rows = min(kPfRows, un.n - m0);
    const bool shared = un.e < 0;
    const int F = shared ? a.Fs : a.F;
    // this lane's weight row: the gate (lanes c < 16) or up (c >= 16) row of
    // SwiGLU column col; 32-bit offsets from per-lane bases (an expert's
    // weights are far below 4 GiB)
    const int col = ct * 128 + 16 * wave + (c & 15);
    gchar_t *gq = uniform_gptr(shared ? a.sgq : a.gq);
    gchar_t *uq = uniform_gptr(shared ? a.suq : a.uq);
    gchar_t *gsc = uniform_gptr(shared ? a.sgs : a.gs);
    gchar_t *usc = uniform_gptr(shared ? a.sus : a.us);
    gchar_t *wq = up_lane ? uq : gq;
    gchar_t *wsc = up_lane ? usc : gsc;
    const uint32_t row0 = static_cast<uint32_t>((shared ? 0 : un.e) * F + col);
    uint32_t woff = row0 * (nblk * 16) + 16 * h, soff = row0 * (nblk * 2);

    // A staging: thread t owns piece t % 16 of rows t / 16 + 32 i.  Rows
    // past the tile's end read token 0's row: their products land in
    // accumulator rows that are never stored (every row of an MFMA result
    // depends on its own A row only), and the requests stay unconditional.
    gchar_t *xg = uniform_gptr(a.x);
    uint32_t xoff[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = (tid >> 4) + 32 * i;
      int t = 0;
      if (r < rows) {
        const int rr = un.r0 + m0 + r;
        t = shared ? rr : (a.row_tok ? a.row_tok[rr] : rr);
        t = t < 0 ? 0 : (t >= T ? T - 1 : t);
      }
      xoff[i] = static_cast<uint32_t>(t) * (2 * H) + 16 * pc;
    }
    auto load_a = [&](int s, uint4(&v)[2]) {
#pragma unroll
      for (int i = 0; i < 2; ++i) v[i] = load16_g(xg + (xoff[i] + 256u * s));
    };
    auto store_a = [&](int buf, const uint4(&v)[2]) {
      // pair-permuted, in fp16
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const u32x4_t pp = pair_permute(v[i]);
        as[buf][(tid >> 4) + 32 * i][pc] = make_uint4(bf16x2_to_f16x2(pp.x), bf16x2_to_f16x2(pp.y),
                                                      bf16x2_to_f16x2(pp.z), bf16x2_to_f16x2(pp.w));
      }
    };
    auto load_b = [&](int s, uint4(&w)[2], u32x2_t &sc) {
      // blocks 4 s + 2 i + h; the four block scales of the step
#pragma unroll
      for (int i = 0; i < 2; ++i) w[i] = load16_g(wq + (woff + 64u * s + 32u * i));
      sc = *reinterpret_cast<gu2_t *>(wsc + (soff + 8u * s));
    };

    f32x16_t acc[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) acc[mt] = zero16();
    uint4 av[2][2];  // A rows of the next two steps, slot s & 1
    uint4 bw[4][2];  // weight chunks, slot s & 3
    u32x2_t bs[4];   // their block scales
    // B(0), A(0), B(1..3), A(1): once A(0) has arrived, B(0) has too (the
    // counter of outstanding loads drains in order)
    load_b(0, bw[0], bs[0]);
    load_a(0, av[0]);
    load_b(1, bw[1], bs[1]);
    load_b(2, bw[2], bs[2]);
    load_b(3, bw[3], bs[3]);
    load_a(1, av[1]);
    store_a(0, av[0]);
    lds_barrier();
    with_msub2((rows + 31) >> 5, [&](auto msc) __attribute__((always_inline)) {
      constexpr int MS = decltype(msc)::value;
      auto step = [&](int s, auto slc) __attribute__((always_inline)) {
        constexpr int sl = decltype(slc)::value;
        pin_u32(woff);
        pin_u32(soff);
#pragma unroll
        for (int i = 0; i < 2; ++i) pin_u32(xoff[i]);
        // unconditional (clamped) requests keep the register slots out of
        // scratch memory; past the end they re-read the last step
        load_a(min(s + 2, KS - 1), av[sl & 1]);
        // kept at the top of the step: two steps of latency for the gather
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < 2; ++i) half_exchange(bw[sl][i]);
#pragma unroll
        for (int t8 = 0; t8 < 8; ++t8) {
          // k 16 t8 .. 16 t8 + 15 of the step: block 2 i + (t >> 1)
          const int i = t8 >> 2, t = t8 & 3;
          const u32x4_t B =
              dequant_f16_pairs(word(bw[sl][i], t), bs[sl].x, bs[sl].y, 2 * i + (t >> 1));
          uint4 Av[MS];
#pragma unroll
          for (int mt = 0; mt < MS; ++mt) Av[mt] = as[sl & 1][32 * mt + c][2 * t8 + h];
#pragma unroll
          for (int mt = 0; mt < MS; ++mt) {
            const u32x4_t A = {Av[mt].x, Av[mt].y, Av[mt].z, Av[mt].w};
            acc[mt] = mfma32_f16(A, B, acc[mt]);
          }
        }
        load_b(min(s + 4, KS - 1), bw[sl], bs[sl]);
        // the weight requests go out before the wait for the A rows below
        __builtin_amdgcn_sched_barrier(0);
        store_a((sl & 1) ^ 1, av[(sl & 1) ^ 1]);  // unconditional: no branch inside the step
        lds_barrier();
      };
      for (int s = 0; s < KS; s += 4) {
        step(s, IntC<0>{});
        step(s + 1, IntC<1>{});
        step(s + 2, IntC<2>{});
        step(s + 3, IntC<3>{});
      }
    });
    // SwiGLU into LDS (the A buffers are free now).  Lane (c, h) holds
    // accumulator j of rows 32 mt + (j & 3) + 8 (j >> 2) + 4 h, gate (c < 16)
    // or up (c >= 16) of SwiGLU column c & 15; swapping register j with
    // j + 8 between the two 16-lane halves of each 32-lane row gives lanes
    // c < 16 gate and up of value j and lanes c >= 16 those of value j + 8.
    // The values are rounded once to fp16 (one plane: the down GEMM's A
    // operand as it is).  Rows [64][128 + 8 pad]; rows past the tile's end
    // hold finite values that are never stored.
    uint16_t *st = reinterpret_cast<uint16_t *>(&as[0][0][0]);
    constexpr int kStRow = 136;
    static_assert(kPfRows * kStRow * 2 <= sizeof(as), "SwiGLU staging must fit the A buffers");
    const int cl = act_pos<MOE_W_INT4_B32>(16 * wave + (c & 15));  // tiles start at multiples of 8
    const int rbase = (up_lane ? 16 : 0) + 4 * h;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int jj = 0; jj < 8; jj += 2) {
        // rows r and r + 1 converted in pairs
        const int r = 32 * mt + (jj & 3) + 8 * (jj >> 2) + rbase;
        float v[2];
#pragma unroll
        for (int d = 0; d < 2; ++d) {
          const auto gu = __builtin_amdgcn_permlane16_swap(__float_as_uint(acc[mt][jj + d]),
                                                           __float_as_uint(acc[mt][jj + d + 8]), false, false);
          const float gv = __uint_as_float(gu[0]), uv = __uint_as_float(gu[1]);
          v[d] = gv * __builtin_amdgcn_rcpf(1.f + __expf(-gv)) * uv;
        }
        const f32x2v_t vv = {v[0], v[1]};
        const uint32_t hv = __builtin_bit_cast(uint32_t, __builtin_convertvector(vv, f16x2_t));
        st[r * kStRow + cl] = static_cast<uint16_t>(hv);
        st[(r + 1) * kStRow + cl] = static_cast<uint16_t>(hv >> 16);
      }
    lds_barrier();
    // 16-byte stores of whole row segments: piece (row, 16 of them)
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      const int idx = tid + kGmThreads * k2;
      const int r = idx >> 4, pcs = idx & 15;
      if (r < rows) {
        const uint4 v = *reinterpret_cast<const uint4 *>(st + r * kStRow + 8 * pcs);
        const int rr = m0 + r;
        const size_t off = shared ? static_cast<size_t>(a.n_rows) * a.F + static_cast<size_t>(rr) * a.Fs
                                  : static_cast<size_t>(un.r0 + rr) * a.F;
        uint16_t *arow = reinterpret_cast<uint16_t *>(a.act + off);
        *reinterpret_cast<uint4 *>(arow + ct * 128 + 8 * pcs) = v;
      }
    }
    lds_barrier();  // the next item's first A tile reuses the buffers
  }
}

// ------------------------------------------------ gate/up, 128-row items
// The layer's gate/up GEMM once its router GEMM has written x in fp16
// operand form (a.x16), with the workspace's item queues (a.queue: nine
// words that are zero between calls).  An item is (unit, up to 128 rows, 128
// SwiGLU columns), so that an expert's rows (64 on average for a prefill
// chunk, rarely above 128) share one pass over its weights: each weight is
// dequantized once per expert instead of once per 64 rows, and a step
// carries up to four 32-row tiles of matrix work per dequantized chunk.
// Blocks take items from their XCD's queue (the shared expert's, the
// largest, first), so that they finish together although items differ in
// size.
// The x rows and the weight chunks go from global memory straight into LDS
// (no registers), two steps ahead, into three buffers each: each x row's
// sixteen 16-byte pieces are stored at slot piece ^ (row & 15), each weight
// row's four blocks at slot block ^ ((row >> 2) & 3), so that the MFMA
// operand reads (16 rows at one piece, or one word of 16 rows) meet every
// LDS bank once.  The weight loads cover 64 contiguous bytes of 16 rows
// each, half the cache lines per request of per-lane register loads.
constexpr int kG2Rows = 128;
constexpr int kG2Queues = 8;  // item queues, one per XCD; the grid is a multiple of this

// Requests one k-step's loads issue in gateup_gemm128_kernel: the A tiles
// (ms) and two weight chunks.
constexpr int g2_requests(int, int ms) { return ms + 2; }

// The unit table of a layer call for the 128-row gate/up kernel: the shared
// expert first, then the experts with rows (offsets[e + 1] > offsets[e]) in
// index order, from one read of the offsets (no dependent reads of the
// active list).  (Ordering the experts by tile count instead, largest first,
// measured 6 us slower.)  Needs n_experts <= kGmMaxUnits - 1.
MOE_DEV int gm_units_from_offsets(const FfnArgs &a, GmUnits &G, int *scratch, int (*cnt)[4]) {
  static_assert(kGmThreads >= kGmMaxUnits, "one unit per thread");
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int E = a.n_experts;
  const int sh = a.Fs > 0 ? 1 : 0;
  int r0 = 0, n = 0;
  if (tid < E) {
    r0 = a.offsets[tid];
    n = a.offsets[tid + 1] - r0;
  }
  // class 0: rows; 4: none (one class: index order)
  const int cls = (tid < E && n > 0) ? 0 : 4;
  uint64_t mine = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint64_t m = __ballot(cls == k);
    if (k == cls) mine = m;
    if (lane == 0) cnt[wave][k] = __popcll(m);
  }
  lds_barrier();
  int n_routed = 0, pos = 0;
#pragma unroll
  for (int w = 0; w < kGmThreads / 64; ++w)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int v = cnt[w][k];
      n_routed += v;
      pos += (k < cls || (k == cls && w < wave)) ? v : 0;
    }
  if (cls < 4) {
    pos += __popcll(mine & ((1ull << lane) - 1));
    G.e[sh + pos] = tid;
    G.r0[sh + pos] = r0;
    G.n[sh + pos] = n;
  }
  if (sh && tid == 0) {
    G.e[0] = -1;
    G.r0[0] = 0;
    G.n[0] = a.T;
  }
  const int n_units = sh + n_routed;
  lds_barrier();
  int c = 0;
  if (tid < n_units) c = (G.n[tid] + kG2Rows - 1) / kG2Rows;
  int inc = c;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(inc, off);
    if (lane >= off) inc += o;
  }
  if (lane == 63) scratch[wave] = inc;
  lds_barrier();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += scratch[w];
  base += inc - c;
  if (tid <= n_units) G.pre[tid] = base;
  lds_barrier();
  return n_units;
}

template <int KS>
__global__ void __launch_bounds__(kGmThreads, 2) gateup_gemm128_kernel(FfnArgs a) {
  static_assert(KS == 16, "the k loop is unrolled over sixteen steps");
  // three A buffers ([kG2Rows][16] pieces) and three weight buffers (the
  // item's 256 weight rows x four 16-byte blocks), two steps ahead: separate
  // arrays, so that the compiler sees that the LDS reads of a step do not
  // touch the buffers its direct loads are filling
  __shared__ uint4 g2_a0[kG2Rows * 16], g2_a1[kG2Rows * 16], g2_a2[kG2Rows * 16];
  __shared__ uint4 g2_b0[256 * 4], g2_b1[256 * 4], g2_b2[256 * 4];
  __shared__ GmUnits units;
  __shared__ int scratch[kGmThreads / 64];
  __shared__ int class_cnt[kGmThreads / 64][4];
  __shared__ int next_item;
  constexpr int nblk = 4 * KS;  // 32-element blocks per weight row
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int c = lane & 31, h = lane >> 5;
  const bool up_lane = c >= 16;
  const int T = a.T;
  const int H = 128 * KS;
  const int n_units = gm_units_from_offsets(a, units, scratch, class_cnt);
  const int col_tiles = a.F / 128;
  // XCD-aware queues: block b runs on XCD b mod 8 and takes items from
  // queue b mod 8, which holds the row tiles j = b mod 8 (mod 8), each row
  // tile's column tiles in a row, so that the column tiles of a row tile run
  // at about the same time on one XCD and share its L2 for their x rows
  const int xq = blockIdx.x & (kG2Queues - 1);
  const int row_tiles = units.pre[n_units];
  const int n_items = (row_tiles > xq ? (row_tiles - xq + kG2Queues - 1) / kG2Queues : 0) * col_tiles;
  auto abuf = [&](int b, int r) __attribute__((always_inline)) {
    return (b == 0 ? g2_a0 : b == 1 ? g2_a1 : g2_a2) + r * 16;
  };
  auto bbuf = [&](int b) __attribute__((always_inline)) { return b == 0 ? g2_b0 : b == 1 ? g2_b1 : g2_b2; };

  for (;;) {
    if (tid == 0) next_item = static_cast<int>(atomicAdd(&a.queue[xq], 1u));
    lds_barrier();
    const int item = next_item;
    if (item >= n_items) break;
    const int jl = item / col_tiles;
    const int ct = item - jl * col_tiles;
    const int j = kG2Queues * jl + xq;
    const int u = pf_find(units.pre, n_units, j);
    const PfUnit un = gm_unit(units, u);
    const int m0 = (j - units.pre[u]) * kG2Rows;
    const int rows = min(kG2Rows, un.n - m0);
    const bool shared = un.e < 0;
    const int F = shared ? a.Fs : a.F;
    gchar_t *gq = uniform_gptr(shared ? a.sgq : a.gq);
    gchar_t *uq = uniform_gptr(shared ? a.suq : a.uq);
    gchar_t *gsc = uniform_gptr(shared ? a.sgs : a.gs);
    gchar_t *usc = uniform_gptr(shared ? a.sus : a.us);
    const uint32_t ebase = static_cast<uint32_t>((shared ? 0 : un.e) * F + ct * 128);
    // The weight tile of a step in LDS: row R (0-127 the gate rows of the
    // item's SwiGLU columns, 128-255 their up rows) holds its four blocks at
    // slots p ^ ((R >> 2) & 3), so that the operand reads (16 rows, one word
    // each) meet every bank once.  Direct loads: instruction k of wave w
    // fills rows 32 w + 16 k .. + 15 (waves 0-3 gate, 4-7 up), lane l row
    // 32 w + 16 k + l / 4, slot l % 4.
    gchar_t *bq = wave < 4 ? gq : uq;
    uint32_t boff[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int R = 32 * wave + 16 * k + (lane >> 2);
      const int p = (lane & 3) ^ ((R >> 2) & 3);
      boff[k] = (ebase + static_cast<uint32_t>(R & 127)) * (nblk * 16) + 16 * p;
    }
    // this lane's operand row (the gate (c < 16) or up (c >= 16) row of
    // SwiGLU column 16 wave + c % 16) and its block scales (registers)
    const int Rm = (up_lane ? 128 : 0) + 16 * wave + (c & 15);
    gchar_t *wsc = up_lane ? usc : gsc;
    uint32_t soff = (ebase + static_cast<uint32_t>(16 * wave + (c & 15))) * (nblk * 2);

    // A: instruction i of this wave fills rows 4 (wave + 8 i) .. + 3 of a
    // buffer, lane l row 4 (wave + 8 i) + l / 16, slot l % 16 (piece
    // (l % 16) ^ row % 16).  Rows past the tile's end read token 0's row:
    // their products land in accumulator rows that are never stored.
    gchar_t *xg = uniform_gptr(a.x16);
    uint32_t xoff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * (wave + 8 * i) + (lane >> 4);
      int t = 0;
      if (r < rows) {
        const int rr = un.r0 + m0 + r;
        t = shared ? rr : (a.row_tok ? a.row_tok[rr] : rr);
        t = t < 0 ? 0 : (t >= T ? T - 1 : t);
      }
      xoff[i] = static_cast<uint32_t>(t) * (2 * H) + 16 * ((lane & 15) ^ (r & 15));
    }
    // the item's block scales, requested first: lane half h holds those of
    // steps 8 h .. 8 h + 7 (64 of its row's 128 bytes); a step takes the
    // holder half's words with one lane swap.  (Register loads of a step's
    // scales beside its direct loads cost about a seventh of the kernel.)
    u32x4_t sreg[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sreg[i] = *reinterpret_cast<gu32x4_t *>(wsc + (soff + 64u * h + 16u * i));
    // the requests of step s into buffer s % 3: its A tiles (MS) and its
    // weight chunks (2 direct loads)
    auto load_step = [&](int s, auto msc) __attribute__((always_inline)) {
      constexpr int MS = decltype(msc)::value;
      const int b = s % 3;
#pragma unroll
      for (int i = 0; i < MS; ++i)
        __builtin_amdgcn_global_load_lds(xg + (xoff[i] + 256u * s),
                                         (__attribute__((address_space(3))) void *)(abuf(b, 4 * (wave + 8 * i))), 16,
                                         0, 0);
#pragma unroll
      for (int k = 0; k < 2; ++k)
        __builtin_amdgcn_global_load_lds(bq + (boff[k] + 64u * s),
                                         (__attribute__((address_space(3))) void *)(bbuf(b) + (32 * wave + 16 * k) * 4),
                                         16, 0, 0);
    };

    f32x16_t acc[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) acc[mt] = zero16();
    with_msub((rows + 31) >> 5, [&](auto msc) __attribute__((always_inline)) {
      constexpr int MS = decltype(msc)::value;
      // steps 0 and 1; the wait leaves step 1's requests pending (the waits
      // count requests in issue order, so each group is pinned)
      load_step(0, msc);
      __builtin_amdgcn_sched_barrier(0);
      load_step(1, msc);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(g2_requests(1, MS)));
      lds_barrier();
      auto step = [&](auto sc) __attribute__((always_inline)) {
        constexpr int s = decltype(sc)::value;
        constexpr int b = s % 3;
        pin_u32(soff);
#pragma unroll
        for (int i = 0; i < 4; ++i) pin_u32(xoff[i]);
#pragma unroll
        for (int k = 0; k < 2; ++k) pin_u32(boff[k]);
        // two steps ahead (clamped: past the end it re-reads the last step,
        // the same bytes into the same buffer)
        constexpr int ahead = s + 2 < KS ? s + 2 : KS - 1;
        load_step(ahead, msc);
        __builtin_amdgcn_sched_barrier(0);
        const uint32_t *brow = reinterpret_cast<const uint32_t *>(bbuf(b) + Rm * 4);
        const int rsw = (Rm >> 2) & 3;
        const u32x4_t &sq = sreg[(s & 7) >> 1];
        const auto sw01 = __builtin_amdgcn_permlane32_swap((s & 1) ? sq.z : sq.x, (s & 1) ? sq.z : sq.x, false, false);
        const auto sw23 = __builtin_amdgcn_permlane32_swap((s & 1) ? sq.w : sq.y, (s & 1) ? sq.w : sq.y, false, false);
        // [0]: the lower half's word in every lane, [1]: the upper half's
        const uint32_t s01 = s < 8 ? sw01[0] : sw01[1], s23 = s < 8 ? sw23[0] : sw23[1];
#pragma unroll
        for (int t8 = 0; t8 < 8; ++t8) {
          // k 16 t8 .. 16 t8 + 15 of the step: block t8 / 2, word 2 (t8 % 2) + h
          const int p = t8 >> 1;
          const uint32_t w = brow[4 * (p ^ rsw) + 2 * (t8 & 1) + h];
          const u32x4_t B = dequant_f16_pairs(w, s01, s23, p);
          const int slot = (2 * t8 + h) ^ (c & 15);
          uint4 Av[MS];
#pragma unroll
          for (int mt = 0; mt < MS; ++mt) Av[mt] = abuf(b, 32 * mt + c)[slot];
#pragma unroll
          for (int mt = 0; mt < MS; ++mt) {
            const u32x4_t A = {Av[mt].x, Av[mt].y, Av[mt].z, Av[mt].w};
            acc[mt] = mfma32_f16(A, B, acc[mt]);
          }
        }
        // step s + 1 has landed once at most step s + 2's requests are pending
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(g2_requests(ahead, MS)));
        lds_barrier();
      };
      step(IntC<0>{});
      step(IntC<1>{});
      step(IntC<2>{});
      step(IntC<3>{});
      step(IntC<4>{});
      step(IntC<5>{});
      step(IntC<6>{});
      step(IntC<7>{});
      step(IntC<8>{});
      step(IntC<9>{});
      step(IntC<10>{});
      step(IntC<11>{});
      step(IntC<12>{});
      step(IntC<13>{});
      step(IntC<14>{});
      step(IntC<15>{});
    });
    // the clamped requests still in flight write into the buffers: let them
    // land before the staging below reuses the memory
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    lds_barrier();
    // SwiGLU into LDS, rounded once to fp16 (as in gateup_gemm_kernel):
    // swapping register j with j + 8 between the 16-lane halves of each
    // 32-lane row gives lanes c < 16 gate and up of value j and lanes
    // c >= 16 those of value j + 8.  Rows [128][128 + 8 pad], rows 0-63 in
    // the first A buffer and 64-127 in the second.
    uint16_t *st0 = reinterpret_cast<uint16_t *>(g2_a0), *st1 = reinterpret_cast<uint16_t *>(g2_a1);
    constexpr int kStRow = 136;
    static_assert(64 * kStRow * 2 <= sizeof(g2_a0), "SwiGLU staging must fit the A buffers");
    const int cl = act_pos<MOE_W_INT4_B32>(16 * wave + (c & 15));  // tiles start at multiples of 8
    const int rbase = (up_lane ? 16 : 0) + 4 * h;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int jj = 0; jj < 8; jj += 2) {
        const int r = 32 * mt + (jj & 3) + 8 * (jj >> 2) + rbase;
        float v[2];
#pragma unroll
        for (int d = 0; d < 2; ++d) {
          const auto gu = __builtin_amdgcn_permlane16_swap(__float_as_uint(acc[mt][jj + d]),
                                                           __float_as_uint(acc[mt][jj + d + 8]), false, false);
          const float gv = __uint_as_float(gu[0]), uv = __uint_as_float(gu[1]);
          v[d] = gv * __builtin_amdgcn_rcpf(1.f + __expf(-gv)) * uv;
        }
        const f32x2v_t vv = {v[0], v[1]};
        const uint32_t hv = __builtin_bit_cast(uint32_t, __builtin_convertvector(vv, f16x2_t));
        uint16_t *st = mt < 2 ? st0 : st1;
        const int rl = r & 63;
        st[rl * kStRow + cl] = static_cast<uint16_t>(hv);
        st[(rl + 1) * kStRow + cl] = static_cast<uint16_t>(hv >> 16);
      }
    lds_barrier();
    // 16-byte stores of whole row segments: piece (row, 16 of them)
#pragma unroll
    for (int k2 = 0; k2 < 4; ++k2) {
      const int idx = tid + kGmThreads * k2;
      const int r = idx >> 4, pcs = idx & 15;
      if (r < rows) {
        const uint4 v = *reinterpret_cast<const uint4 *>((k2 < 2 ? st0 : st1) + (r & 63) * kStRow + 8 * pcs);
        const int rr = m0 + r;
        const size_t off = shared ? static_cast<size_t>(a.n_rows) * a.F + static_cast<size_t>(rr) * a.Fs
                                  : static_cast<size_t>(un.r0 + rr) * a.F;
        uint16_t *arow = reinterpret_cast<uint16_t *>(a.act + off);
        *reinterpret_cast<uint4 *>(arow + ct * 128 + 8 * pcs) = v;
      }
    }
    lds_barrier();  // the next item's first A tiles reuse the memory
  }
  // the last block out leaves the queue words zero for the next call
  if (tid == 0) {
    __threadfence();
    if (atomicAdd(&a.queue[kG2Queues], 1u) == gridDim.x - 1) {
#pragma unroll
      for (int q = 0; q <= kG2Queues; ++q) atomicExch(&a.queue[q], 0u);
    }
  }
}

// ------------------------------------------------ down, operands through LDS
// The down GEMM with both operands staged by direct loads, one step ahead,
// in two buffers each (LDS 64 KB a block: two blocks a compute unit): the
// act rows (64 rows x 256 bytes a step, pieces swizzled by row as in
// gateup_gemm128_kernel) and the weight chunks of the item's 256 output
// columns (16 rows of 64 contiguous bytes a request, blocks swizzled by
// row); the block scales are register loads.  The products leave the
// accumulators directly (32 lanes: 32 consecutive columns of one row).
template <int KS, bool F16>
__global__ void __launch_bounds__(kGmThreads, 4) down_gemm_kernel(FfnArgs a) {
  static_assert(KS == 4, "four k-steps");
  __shared__ uint4 dn_a0[kPfRows * 16], dn_a1[kPfRows * 16];
  __shared__ uint4 dn_b0[256 * 4], dn_b1[256 * 4];
  __shared__ GmUnits units;
  __shared__ int scratch[kGmThreads / 64];
  __shared__ float wrow[kPfRows];
  constexpr int nblk = 4 * KS;  // 32-element blocks per weight row
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int c = lane & 31, h = lane >> 5;
  const int H = a.H;
  const int n_units = gm_units(a, units, scratch);
  const int col_tiles = H / 256;
  const int n_items = units.pre[n_units] * col_tiles;
  auto abuf = [&](int b) __attribute__((always_inline)) { return b == 0 ? dn_a0 : dn_a1; };
  auto bbuf = [&](int b) __attribute__((always_inline)) { return b == 0 ? dn_b0 : dn_b1; };

  // XCD-aware order: the blocks of one XCD (block b runs on XCD b mod 8)
  // take a contiguous run of items per round, so the column tiles of a row
  // tile share that XCD's L2 for their act rows
  const int per_xcd = gridDim.x >> 3;
  const int my_off = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  for (int round = 0; round < n_items; round += gridDim.x) {
    const int item = round + my_off;
    if (item >= n_items) continue;
    const int j = item / col_tiles;
    const int ct = item - j * col_tiles;
    const int u = pf_find(units.pre, n_units, j);
    const PfUnit un = gm_unit(units, u);
    const int m0 = (j - units.pre[u]) * kPfRows;
    const int rows = min(kPfRows, un.n - m0);
    const bool shared = un.e < 0;
    const int F = shared ? a.Fs : a.F;  // == 128 KS
    gchar_t *dq = uniform_gptr(shared ? a.sdq : a.dq);
    gchar_t *dsc = uniform_gptr(shared ? a.sds : a.ds);
    const uint32_t ebase = static_cast<uint32_t>((shared ? 0 : un.e) * H + ct * 256);
    // weights: instruction k of wave w fills tile rows 32 w + 16 k .. + 15,
    // lane l row 32 w + 16 k + l / 4, slot l % 4 (block (l % 4) ^ ((row >> 2) & 3))
    uint32_t boff[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int R = 32 * wave + 16 * k + (lane >> 2);
      boff[k] = (ebase + static_cast<uint32_t>(R)) * (nblk * 16) + 16 * ((lane & 3) ^ ((R >> 2) & 3));
    }
    // act: instruction i of wave w fills rows 4 (w + 8 i) .. + 3, lane l row
    // 4 (w + 8 i) + l / 16, slot l % 16 (piece (l % 16) ^ (row % 16)); the
    // rows are consecutive in the act buffer, 4 bytes a slot element (the
    // fp16 plane in the first half); rows past the tile's end read its first
    gchar_t *ag = uniform_gptr(a.act);
    const uint32_t abase = shared ? static_cast<uint32_t>(a.n_rows * a.F + m0 * a.Fs)
                                  : static_cast<uint32_t>((un.r0 + m0) * a.F);
    uint32_t aoff[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = 4 * (wave + 8 * i) + (lane >> 4);
      aoff[i] = 4 * (abase + static_cast<uint32_t>((r < rows ? r : 0) * F)) + 16 * ((lane & 15) ^ (r & 15));
    }
    // this lane's operand row (output column hcol) and its block scales
    const int Rm = 32 * wave + c;
    const int hcol = ct * 256 + Rm;
    const uint32_t soff = (ebase + static_cast<uint32_t>(Rm)) * (nblk * 2);
    if (tid < kPfRows) {
      const int r = tid < rows ? tid : 0;
      wrow[tid] = shared || !a.row_w ? 1.f : a.row_w[un.r0 + m0 + r];
    }
    // the item's block scales, requested first: lane half h holds those of
    // steps 2 h and 2 h + 1 (16 of its row's 32 bytes), taken by a lane swap
    const u32x4_t sreg = *reinterpret_cast<gu32x4_t *>(dsc + (soff + 16u * h));
    auto load_step = [&](int s) __attribute__((always_inline)) {
      const int b = s & 1;
#pragma unroll
      for (int i = 0; i < 2; ++i)
        __builtin_amdgcn_global_load_lds(ag + (aoff[i] + 256u * s),
                                         (__attribute__((address_space(3))) void *)(abuf(b) + 4 * (wave + 8 * i) * 16),
                                         16, 0, 0);
#pragma unroll
      for (int k = 0; k < 2; ++k)
        __builtin_amdgcn_global_load_lds(dq + (boff[k] + 64u * s),
                                         (__attribute__((address_space(3))) void *)(bbuf(b) + (32 * wave + 16 * k) * 4),
                                         16, 0, 0);
    };

    f32x16_t acc[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) acc[mt] = zero16();
    load_step(0);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    lds_barrier();
    with_msub2((rows + 31) >> 5, [&](auto msc) __attribute__((always_inline)) {
      constexpr int MS = decltype(msc)::value;
      auto step = [&](auto sc) __attribute__((always_inline)) {
        constexpr int s = decltype(sc)::value;
        constexpr int b = s & 1;
        // one step ahead
        if constexpr (s + 1 < KS) load_step(s + 1);
        __builtin_amdgcn_sched_barrier(0);
        const uint32_t *brow = reinterpret_cast<const uint32_t *>(bbuf(b) + Rm * 4);
        const int rsw = (Rm >> 2) & 3;
#pragma unroll
        for (int t8 = 0; t8 < 8; ++t8) {
          const int p = t8 >> 1;
          const uint32_t w = brow[4 * (p ^ rsw) + 2 * (t8 & 1) + h];
          const auto sw01 = __builtin_amdgcn_permlane32_swap((s & 1) ? sreg.z : sreg.x, (s & 1) ? sreg.z : sreg.x,
                                                             false, false);
          const auto sw23 = __builtin_amdgcn_permlane32_swap((s & 1) ? sreg.w : sreg.y, (s & 1) ? sreg.w : sreg.y,
                                                             false, false);
          const u32x4_t B = dequant_f16_pairs(w, s < 2 ? sw01[0] : sw01[1], s < 2 ? sw23[0] : sw23[1], p);
          const int slot = (2 * t8 + h) ^ (c & 15);
          uint4 Av[MS];
#pragma unroll
          for (int mt = 0; mt < MS; ++mt) Av[mt] = abuf(b)[(32 * mt + c) * 16 + slot];
#pragma unroll
          for (int mt = 0; mt < MS; ++mt) {
            const u32x4_t A = {Av[mt].x, Av[mt].y, Av[mt].z, Av[mt].w};
            acc[mt] = mfma32_f16(A, B, acc[mt]);
          }
        }
        // step s + 1 has landed once nothing is pending; after the last
        // step the barrier frees the tiles for the next item
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        lds_barrier();
      };
      step(IntC<0>{});
      step(IntC<1>{});
      step(IntC<2>{});
      step(IntC<3>{});
    });
    // rows of the tile times their routing weights, straight to the output
    // rows (fp32, or rounded once to fp16 with rows_f16): register jj of
    // lane (c, h) is row 32 mt + (jj & 3) + 8 (jj >> 2) + 4 h
    {
      const int orow0 = shared ? a.n_rows + m0 : un.r0 + m0;
      const size_t o0 = static_cast<size_t>(orow0 + 4 * h) * H + hcol;
      if constexpr (F16) {
        _Float16 *op = reinterpret_cast<_Float16 *>(a.rows_out) + o0;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int jj = 0; jj < 16; ++jj) {
            const int R = 32 * mt + (jj & 3) + 8 * (jj >> 2);
            if (R + 4 * h < rows) op[R * H] = static_cast<_Float16>(acc[mt][jj] * wrow[R + 4 * h]);
          }
      } else {
        float *op = a.rows_out + o0;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int jj = 0; jj < 16; ++jj) {
            const int R = 32 * mt + (jj & 3) + 8 * (jj >> 2);
            if (R + 4 * h < rows) op[R * H] = acc[mt][jj] * wrow[R + 4 * h];
          }
      }
    }
    lds_barrier();  // the next item's tiles and row weights reuse the memory
  }
}

// ---------------------------------------------------------- W8A8 variant
//
// int8 activations with int8 row-scaled weights (the W8A8 variant: the
// pages' engines quantise activations to 8 bits at every quantised matrix,
// "Models and backends", How each backend was checked; the B70 prompt path
// multiplies int8 weights by int8 activations, "Strata on an Intel Arc",
// Arc Pro B70: the fused int8 expert path for the prompt).  Every token's
// input and every (token, expert) SwiGLU row is quantised with one symmetric
// scale per row; since the weights carry one scale per row too, both scales
// factor out of the whole reduction: I = sum_k qa[k] qw[k] accumulates
// exactly in int32 on the int8 matrix cores (v_mfma_i32_32x32x32_i8) and
// the epilogue applies d_row * s_col once.
//
// Quantiser (one block per row): amax = max |v|, inv = 127 / amax and
// d = amax / 127 (correctly rounded divisions), q = round-half-even(v * inv)
// (one rounded product), clamped to [-127, 127]; amax = 0 gives q = 0, d = 0.
// Every decision in float32, as the reference statement of the variant.
//
// GEMM tiles.  An item is (unit, up to 128 rows, 128 SwiGLU columns for
// gate/up, 256 output columns for down): with 64 rows an expert on average
// (at most about 90 for uniform routing), one item covers all of an
// expert's rows, so every weight is read once.  Both operands go from
// global memory straight into LDS (direct loads, no registers), two k-steps
// of 128 ahead, into three buffers each, as in gateup_gemm128_kernel: each
// 128-byte row segment's eight 16-byte pieces are stored at slot
// piece ^ (row & 7), so that the operand reads (32 rows at one piece) spread
// over the banks, and every request covers whole 128-byte lines.  Each of
// the 8 waves owns 32 output columns (gate/up: the gate and the up rows of
// 16 SwiGLU columns) for all the item's rows, four 32x32 tiles along M.
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x16_t __attribute__((ext_vector_type(16)));

MOE_DEV i32x16_t mfma_i8(const i32x4_t &a, const i32x4_t &b, const i32x16_t &c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}

constexpr int kQrThreads = 256;
constexpr int kQrMaxPer = 16;  // elements a thread holds: rows of up to 4096

MOE_DEV float qr_value(const uint16_t *p, int i) { return bf16_to_f32(p[i]); }
MOE_DEV float qr_value(const float *p, int i) { return p[i]; }

template <typename In>
__global__ void __launch_bounds__(kQrThreads) quant_rows_kernel(const In *__restrict__ in, int K,
                                                                int8_t *__restrict__ q, float *__restrict__ d) {
  __shared__ float wmax[kQrThreads / 64];
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const In *src = in + static_cast<size_t>(row) * K;
  float v[kQrMaxPer];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < kQrMaxPer; ++i) {
    const int idx = tid + kQrThreads * i;
    v[i] = idx < K ? qr_value(src, idx) : 0.f;
    amax = fmaxf(amax, fabsf(v[i]));
  }
  // block maximum (non-negative floats order as their bit patterns)
  uint32_t m = __float_as_uint(amax);
  m = max(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), 1)));
  m = max(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), 2)));
  m = max(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), 4)));
  m = max(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), 8)));
  m = max(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), 16)));
  m = max(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), 32)));
  if ((tid & 63) == 0) wmax[tid >> 6] = __uint_as_float(m);
  lds_barrier();
  amax = wmax[0];
#pragma unroll
  for (int w = 1; w < kQrThreads / 64; ++w) amax = fmaxf(amax, wmax[w]);
  const float inv = amax > 0.f ? 127.f / amax : 0.f;
  int8_t *dst = q + static_cast<size_t>(row) * K;
#pragma unroll
  for (int i = 0; i < kQrMaxPer; ++i) {
    const int idx = tid + kQrThreads * i;
    if (idx < K) {
      const float r = rintf(v[i] * inv);  // one rounded product, ties to even
      dst[idx] = static_cast<int8_t>(static_cast<int>(fminf(127.f, fmaxf(-127.f, r))));
    }
  }
  if (tid == 0) d[row] = amax > 0.f ? amax / 127.f : 0.f;
}

constexpr int kW8Rows = 128;  // rows per item
constexpr int kW8Step = 128;  // k (bytes of an int8 row) per step
static int pf_grid(int items_upper);

// The W8A8 GEMM.  GATEUP: a[row][f] = silu(g) u with g = I_g dx[t] sg[f]
// (and u alike), the rows' tokens' quantised inputs against the gate and
// up rows f; K = H.  Otherwise (down): rows_out[row][h] = I dA[row] w[row]
// sd[h], the rows' quantised SwiGLU rows against the down rows h; K = F.
// KS = K / 128 steps, unrolled.
template <bool GATEUP, int KS>
__global__ void __launch_bounds__(kGmThreads) w8a8_gemm_kernel(FfnArgs a) {
  // three A buffers (128 rows x eight 16-byte pieces) and three weight
  // buffers (256 rows x eight pieces): separate arrays, so that the
  // compiler sees that the LDS reads of a step do not touch the buffers its
  // direct loads are filling
  __shared__ uint4 w8_a0[kW8Rows * 8], w8_a1[kW8Rows * 8], w8_a2[kW8Rows * 8];
  __shared__ uint4 w8_b0[256 * 8], w8_b1[256 * 8], w8_b2[256 * 8];
  __shared__ GmUnits units;
  __shared__ int scratch[kGmThreads / 64];
  __shared__ float rsc[kW8Rows];  // the row's activation scale (x routing weight for down)
  __shared__ int arow[kW8Rows];   // down: the row's act row (= its output row)
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int c = lane & 31, h = lane >> 5;
  const int T = a.T;
  const int K = kW8Step * KS;
  const int n_units = gm_units<kW8Rows>(a, units, scratch);
  const int NC = GATEUP ? 128 : 256;  // output columns of an item
  const int col_groups = (GATEUP ? a.F : a.H) / NC;
  const int n_items = units.pre[n_units] * col_groups;
  auto abuf = [&](int b) __attribute__((always_inline)) { return b == 0 ? w8_a0 : b == 1 ? w8_a1 : w8_a2; };
  auto bbuf = [&](int b) __attribute__((always_inline)) { return b == 0 ? w8_b0 : b == 1 ? w8_b1 : w8_b2; };
  // this lane's operand row of the weight tile: gate/up: the gate (c < 16)
  // or up (c >= 16) row of SwiGLU column 16 wave + c % 16; down: column
  // 32 wave + c
  const int Rm = GATEUP ? (c >= 16 ? 128 : 0) + 16 * wave + (c & 15) : 32 * wave + c;

  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int j = item / col_groups;
    const int cg = item - j * col_groups;
    const int u = pf_find(units.pre, n_units, j);
    const PfUnit un = gm_unit(units, u);
    const int m0 = (j - units.pre[u]) * kW8Rows;
    const int rows = min(kW8Rows, un.n - m0);
    const bool shared = un.e < 0;
    const int e = shared ? 0 : un.e;
    lds_barrier();  // the previous item's readers of rsc / arow are done
    if (tid < kW8Rows) {
      float sc = 0.f;
      int ar = 0;
      if (tid < rows) {
        const int rr = un.r0 + m0 + tid;  // routed: row index; shared: token
        if (GATEUP) {
          int t = shared ? rr : (a.row_tok ? a.row_tok[rr] : rr);
          t = t < 0 ? 0 : (t >= T ? T - 1 : t);  // memory safety for malformed row lists
          sc = a.dx[t];
          ar = t;
        } else {
          ar = shared ? a.n_rows + rr : rr;
          sc = a.da[ar] * (shared || !a.row_w ? 1.f : a.row_w[rr]);
        }
      }
      rsc[tid] = sc;
      arow[tid] = ar;  // gate/up: the row's token
    }
    lds_barrier();
    // Weight tile rows: instruction k of wave w fills rows 32 w + 8 k + l / 8
    // (gate/up: 0-127 the gate rows of the item's SwiGLU columns, 128-255
    // their up rows), slot l % 8, with piece slot ^ (row & 7).
    gchar_t *bq;
    uint32_t bbase;
    if (GATEUP) {
      const int F = shared ? a.Fs : a.F;
      bq = uniform_gptr(wave < 4 ? (shared ? a.sgq : a.gq) : (shared ? a.suq : a.uq));
      bbase = static_cast<uint32_t>(e * F + cg * 128);
    } else {
      bq = uniform_gptr(shared ? a.sdq : a.dq);
      bbase = static_cast<uint32_t>(e * a.H + cg * 256);
    }
    uint32_t boff[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int R = 32 * wave + 8 * k + (lane >> 3);
      boff[k] = (bbase + static_cast<uint32_t>(GATEUP ? (R & 127) : R)) * K + 16 * ((lane & 7) ^ (R & 7));
    }
    // A rows: instruction i of wave w fills rows 8 (w + 8 i) + l / 8, slot l % 8;
    // rows past the tile's end read the first row (their products land in
    // accumulator rows that are never stored)
    gchar_t *aq = uniform_gptr(GATEUP ? static_cast<const void *>(a.qx) : static_cast<const void *>(a.qa));
    uint32_t aoff[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = 8 * (wave + 8 * i) + (lane >> 3);
      const int src = arow[r < rows ? r : 0];
      aoff[i] = static_cast<uint32_t>(src) * K + 16 * ((lane & 7) ^ (r & 7));
    }
    auto load_step = [&](int s, auto msc) __attribute__((always_inline)) {
      constexpr int MS = decltype(msc)::value;
      const int b = s % 3;
#pragma unroll
      for (int i = 0; i < (MS + 1) / 2; ++i)
        __builtin_amdgcn_global_load_lds(aq + (aoff[i] + static_cast<uint32_t>(kW8Step) * s),
                                         (__attribute__((address_space(3))) void *)(abuf(b) + 8 * 8 * (wave + 8 * i)),
                                         16, 0, 0);
#pragma unroll
      for (int k = 0; k < 4; ++k)
        __builtin_amdgcn_global_load_lds(bq + (boff[k] + static_cast<uint32_t>(kW8Step) * s),
                                         (__attribute__((address_space(3))) void *)(bbuf(b) + 8 * (32 * wave + 8 * k)),
                                         16, 0, 0);
    };

    i32x16_t acc[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mt][r] = 0;
    with_msub((rows + 31) >> 5, [&](auto msc) __attribute__((always_inline)) {
      constexpr int MS = decltype(msc)::value;
      constexpr int G = (MS + 1) / 2 + 4;  // requests a step
      // steps 0 and 1; the wait leaves step 1's requests pending (the waits
      // count requests in issue order, so each group is pinned)
      load_step(0, msc);
      __builtin_amdgcn_sched_barrier(0);
      load_step(1, msc);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(G));
      lds_barrier();
      auto step = [&](auto sc) __attribute__((always_inline)) {
        constexpr int s = decltype(sc)::value;
        constexpr int b = s % 3;
        pin_u32(aoff[0]);
        pin_u32(aoff[1]);
#pragma unroll
        for (int k = 0; k < 4; ++k) pin_u32(boff[k]);
        // two steps ahead (clamped: past the end it re-reads the last
        // step, the same bytes into the same buffer)
        load_step(s + 2 < KS ? s + 2 : KS - 1, msc);
        __builtin_amdgcn_sched_barrier(0);
        const uint4 *brow = bbuf(b) + 8 * Rm;
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) {
          // k 32 t4 .. 32 t4 + 31 of the step: piece 2 t4 + h of the rows
          const int pc = 2 * t4 + h;
          const uint4 bv = brow[pc ^ (Rm & 7)];
          const i32x4_t B = {static_cast<int>(bv.x), static_cast<int>(bv.y), static_cast<int>(bv.z),
                             static_cast<int>(bv.w)};
          uint4 Av[MS];
#pragma unroll
          for (int mt = 0; mt < MS; ++mt) Av[mt] = abuf(b)[8 * (32 * mt + c) + (pc ^ (c & 7))];
#pragma unroll
          for (int mt = 0; mt < MS; ++mt) {
            const i32x4_t A = {static_cast<int>(Av[mt].x), static_cast<int>(Av[mt].y), static_cast<int>(Av[mt].z),
                               static_cast<int>(Av[mt].w)};
            acc[mt] = mfma_i8(A, B, acc[mt]);
          }
        }
        // step s + 1 has landed once at most step s + 2's requests are pending
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(G));
        lds_barrier();
      };
      unrolled_steps(std::make_integer_sequence<int, KS>{}, step);
    });
    // the clamped requests still in flight write into the buffers: let them
    // land before the next item's requests reuse them
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    // epilogue: result (m, n) of a 32x32 tile sits in lane n + 32 ((m / 4) % 2),
    // register 4 (m / 8) + m % 4
    if (GATEUP) {
      // scaled products; then register j swapped with j + 8 between the
      // 16-lane halves of each 32-lane row: lanes c < 16 hold gate and up of
      // value j, lanes c >= 16 those of value j + 8
      const int F = shared ? a.Fs : a.F;
      const size_t srow = static_cast<size_t>(e) * F + cg * 128 + 16 * wave + (c & 15);
      const float sl = static_cast<const float *>(c >= 16 ? (shared ? a.sus : a.us) : (shared ? a.sgs : a.gs))[srow];
      const int rbase = (c >= 16 ? 16 : 0) + 4 * h;
      const int col = cg * 128 + 16 * wave + (c & 15);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const int rlo = 32 * mt + 8 * (jj >> 2) + 4 * h + (jj & 3);  // row of register jj
          const int rhi = rlo + 16;                                    // row of register jj + 8
          const float vlo = static_cast<float>(acc[mt][jj]) * rsc[rlo] * sl;
          const float vhi = static_cast<float>(acc[mt][jj + 8]) * rsc[rhi] * sl;
          const auto gu = __builtin_amdgcn_permlane16_swap(__float_as_uint(vlo), __float_as_uint(vhi), false, false);
          const float gv = __uint_as_float(gu[0]), uv = __uint_as_float(gu[1]);
          const int r = 32 * mt + 8 * (jj >> 2) + (jj & 3) + rbase;
          if (r < rows) {
            const int rr = m0 + r;
            const size_t ar = shared ? static_cast<size_t>(a.n_rows) + rr : static_cast<size_t>(un.r0) + rr;
            a.act[ar * a.F + col] = gv / (1.f + expf(-gv)) * uv;
          }
        }
    } else {
      const int col = cg * 256 + 32 * wave + c;
      const float sd = static_cast<const float *>(shared ? a.sds : a.ds)[static_cast<size_t>(e) * a.H + col];
      _Float16 *o16 = reinterpret_cast<_Float16 *>(a.rows_out);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r16 = 0; r16 < 16; ++r16) {
          const int m = 32 * mt + 8 * (r16 >> 2) + 4 * h + (r16 & 3);
          const float v = static_cast<float>(acc[mt][r16]) * rsc[m] * sd;
          const size_t o = static_cast<size_t>(arow[m]) * a.H + col;
          if (m < rows) {
            if (a.rows_f16)
              o16[o] = static_cast<_Float16>(v);  // rounded once (rows_f16)
            else
              a.rows_out[o] = v;
          }
        }
    }
  }
}

bool w8a8_ok(const FfnArgs &a) {
  const int units = (a.Fs > 0 ? 1 : 0) + (a.offsets ? a.max_units : 1);
  auto steps_ok = [](int k) { return k == 2 * kW8Step || k == 4 * kW8Step || k == 8 * kW8Step || k == 16 * kW8Step; };
  return a.fmt == MOE_W_INT8_ROW && (a.Fs == 0 || a.Fs == a.F) && steps_ok(a.H) && steps_ok(a.F) && a.H % 256 == 0 &&
         units <= kGmMaxUnits && a.qx && a.dx && a.qa && a.da;
}

// Blocks of a W8A8 GEMM launch: one per compute unit (its LDS holds one
// block), fewer for fewer items.
static int w8_grid(int items_upper) {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
  }
  return items_upper < 1 ? 1 : (items_upper < cus ? items_upper : cus);
}

template <bool GATEUP>
static hipError_t launch_w8a8_gemm(const FfnArgs &a, hipStream_t s, const LaunchEvents &ev) {
  const int units = (a.Fs > 0 ? 1 : 0) + (a.offsets ? a.max_units : 1);
  const int tiles = (a.n_rows + kW8Rows - 1) / kW8Rows + units + (a.Fs > 0 ? (a.T + kW8Rows - 1) / kW8Rows : 0);
  const int K = GATEUP ? a.H : a.F;
  const int grid = w8_grid(tiles * (GATEUP ? a.F / 128 : a.H / 256));
  switch (K / kW8Step) {
    case 16:
      return launch_kernel(w8a8_gemm_kernel<GATEUP, 16>, dim3(grid), dim3(kGmThreads), 0, s, ev, a);
    case 8:
      return launch_kernel(w8a8_gemm_kernel<GATEUP, 8>, dim3(grid), dim3(kGmThreads), 0, s, ev, a);
    case 4:
      return launch_kernel(w8a8_gemm_kernel<GATEUP, 4>, dim3(grid), dim3(kGmThreads), 0, s, ev, a);
    default:
      return launch_kernel(w8a8_gemm_kernel<GATEUP, 2>, dim3(grid), dim3(kGmThreads), 0, s, ev, a);
  }
}

hipError_t launch_w8a8(const FfnArgs &a, hipStream_t s, const LaunchEvents &ev_gu, const LaunchEvents &ev_dn) {
  if (!w8a8_ok(a)) return hipErrorInvalidValue;
  // every token's input, quantised per row
  quant_rows_kernel<uint16_t><<<a.T, kQrThreads, 0, s>>>(a.x, a.H, a.qx, a.dx);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_w8a8_gemm<true>(a, s, ev_gu);
  if (e != hipSuccess) return e;
  // every SwiGLU row (routed, then the shared expert's), quantised per row
  const int rows_all = a.n_rows + (a.Fs > 0 ? a.T : 0);
  quant_rows_kernel<float><<<rows_all, kQrThreads, 0, s>>>(a.act, a.F, a.qa, a.da);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_w8a8_gemm<false>(a, s, ev_dn);
}

// ----------------------------------------------------------------- launches

bool prefill_ok(const FfnArgs &a) {
  const int units = (a.Fs > 0 ? 1 : 0) + (a.offsets ? a.max_units : 1);
  const bool many = a.path == kPathPrefill || (a.path == kPathAuto && a.T > kFusedTokens);
  return a.fmt == MOE_W_INT4_B32 && many && (a.Fs == 0 || a.Fs == a.F) && a.H % 128 == 0 &&
         a.F % 128 == 0 && a.F % kPfCols == 0 && a.H % kPfCols == 0 && units <= kPfMaxUnits;
}

static int pf_grid(int items_upper) {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
  }
  const int cap = 3 * cus;  // the blocks resident at once (three per compute unit)
  return items_upper < 1 ? 1 : (items_upper < cap ? items_upper : cap);
}

// Upper bound of the row tiles: every routed row tile plus one partial tile
// per unit, plus the shared expert's.
static int pf_tiles_upper(const FfnArgs &a) {
  const int units = a.offsets ? a.max_units : 1;
  return (a.n_rows + kPfRows - 1) / kPfRows + units + (a.Fs > 0 ? (a.T + kPfRows - 1) / kPfRows : 0);
}

// Blocks of a GEMM launch: per_cu per compute unit (fewer when there are
// fewer items), a multiple of the 8 XCDs (the item order relies on it).
static int gm_grid(int items_upper, int per_cu) {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
  }
  const int cap = per_cu * cus;
  const int g = items_upper < 1 ? 1 : (items_upper < cap ? items_upper : cap);
  return (g + 7) & ~7;
}

static bool gm_units_fit(const FfnArgs &a) {
  return (a.Fs > 0 ? 1 : 0) + (a.offsets ? a.max_units : 1) <= kGmMaxUnits;
}

// The pipelined GEMMs run as a pair (the gate/up one hands the down one its
// SwiGLU rows as one fp16 plane; the generic kernels use bf16 hi and lo).
static bool gm_pair_ok(const FfnArgs &a) { return a.H == 128 * 16 && a.F == 128 * 4 && gm_units_fit(a); }

hipError_t launch_gateup_prefill(const FfnArgs &a, hipStream_t s) {
  if (gm_pair_ok(a) && a.x16 && a.queue && a.offsets && a.n_experts < kGmMaxUnits) {
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) {
      int v = 0;
      if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
    }
    // every queue needs blocks: a multiple of kG2Queues
    const int grid = (cus + kG2Queues - 1) / kG2Queues * kG2Queues;
    return launch_kernel(gateup_gemm128_kernel<16>, dim3(grid), dim3(kGmThreads), 0, s, a.ev, a);
  }
  if (gm_pair_ok(a)) {
    return launch_kernel(gateup_gemm_kernel<16>, dim3(gm_grid(pf_tiles_upper(a) * (a.F / 128), 1)), dim3(kGmThreads), 0,
                         s, a.ev, a);
  }
  return launch_kernel(gateup_prefill_kernel, dim3(pf_grid(pf_tiles_upper(a) * (a.F / kPfCols))), dim3(kPfThreads), 0,
                       s, a.ev, a);
}

bool down_rows_f16_ok(const FfnArgs &a) { return prefill_ok(a) && gm_pair_ok(a); }

hipError_t launch_down_prefill(const FfnArgs &a, hipStream_t s) {
  if (gm_pair_ok(a)) {
    const dim3 grid(gm_grid(pf_tiles_upper(a) * (a.H / 256), 2));
    if (a.rows_f16) return launch_kernel(down_gemm_kernel<4, true>, grid, dim3(kGmThreads), 0, s, a.ev, a);
    return launch_kernel(down_gemm_kernel<4, false>, grid, dim3(kGmThreads), 0, s, a.ev, a);
  }
  return launch_kernel(down_prefill_kernel, dim3(pf_grid(pf_tiles_upper(a) * (a.H / kPfCols))), dim3(kPfThreads), 0,
                       s, a.ev, a);
}

}  // namespace moe
