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
// Arithmetic as in the decode kernels (expert_mfma.hip): the int4 weights
// enter the MFMA as the exact bfloat16 values 128 + nibble = q + 136, the
// other operand is exact (x in bf16; the SwiGLU output as bf16 hi + lo), the
// fp32 accumulator input of each 32-element block is -136 * sum(other
// operand over the block) (computed while the operand tile is staged), and
// the block's fp16 scale is applied with an fp32 FMA.
//
// Tiles.  An item is (unit, 64 rows, 64 output columns); a block of 4 waves
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
template <int NT = kPfThreads>
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
      c = x.n > 0 ? (x.n + kPfRows - 1) / kPfRows : 0;
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
// Down (F = 512: four steps) keeps the weights of the next two steps and the
// A rows of the next one in flight, two blocks per compute unit.  Gate/up
// (H = 2048: sixteen steps) runs one block per compute unit with 256
// registers a lane and keeps the weights of the next four steps and the A
// rows of the next two in flight, and reads a block's A fragments from LDS
// together before its MFMAs (with 128 registers hipcc read and waited for
// each fragment right before its MFMA; measured: 202 against 216 us for the
// prefill chunk).  Tiles are wider than the generic
// kernels' (128 SwiGLU columns for gate/up, 256 output columns for down, 64
// rows), each wave owning two 16-column weight tiles against the 16-row
// tiles of A.  Unlike the generic kernels, these multiply in fp16: each
// weight is dequantized once per item to the fp16 value q s (rounded once,
// relative error at most 2^-11) and the A rows are staged in fp16 (x, and
// the hi and lo parts of the SwiGLU rows, are bf16 values, exact in fp16
// within its normal range), so the products accumulate in the matrix core
// with no sum correction and no per-block scaling on the vector unit.
//
// The k loop is instantiated once per number of 16-row tiles that hold rows
// (1..4), chosen per item: no matrix-core instruction sits under a branch.
// (With the tile count as a branch inside the loop, hipcc left an MFMA
// result read by a VALU instruction right after the branch without the
// wait states the matrix core needs, and those reads saw stale registers.)

typedef __attribute__((address_space(1))) const u32x2_t gu2_t;


// An empty volatile statement that takes the value in registers: volatile
// statements keep their order, so each scaled accumulation happens where it
// is written, instead of every product of a step being computed first and
// held (which spills).
MOE_DEV void pin(f32x4_t &v) { __asm__ volatile("" : "+v"(v)); }
// The same for a 32-bit offset: the addresses derived from it are then
// computed where they are used rather than hoisted out of the k loop and
// kept live (which spills, and a spill reload waits for every load).
MOE_DEV void pin_u32(uint32_t &v) { __asm__ volatile("" : "+v"(v)); }

template <int V>
struct IntC {
  static constexpr int value = V;
};

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
    c = x.n > 0 ? (x.n + kPfRows - 1) / kPfRows : 0;
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
  static_assert(KS % 2 == 0, "the k loop runs over pairs of steps");
  __shared__ uint4 as[2][kPfRows][17];  // x rows of the tile, pair-permuted fp16, one k-step
  __shared__ GmUnits units;
  __shared__ int scratch[kGmThreads / 64];
  constexpr int nblk = 4 * KS;  // 32-element blocks per weight row
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int n = lane & 15, g = lane >> 4;
  const int T = a.T;
  const int H = 128 * KS;
  const int n_units = gm_units(a, units, scratch);
  const int col_tiles = a.F / 128;
  const int n_items = units.pre[n_units] * col_tiles;
  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
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
    // this lane's weight rows: the gate (q = 0) and up (q = 1) rows of SwiGLU
    // column col; 32-bit offsets from block-uniform bases (an expert's
    // weights are far below 4 GiB)
    const int col = ct * 128 + 16 * wave + n;
    gchar_t *gq = uniform_gptr(shared ? a.sgq : a.gq);
    gchar_t *uq = uniform_gptr(shared ? a.suq : a.uq);
    gchar_t *gsc = uniform_gptr(shared ? a.sgs : a.gs);
    gchar_t *usc = uniform_gptr(shared ? a.sus : a.us);
    const uint32_t row0 = static_cast<uint32_t>((shared ? 0 : un.e) * F + col);
    uint32_t woff = row0 * (nblk * 16) + 16 * g, soff = row0 * (nblk * 2);

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
    auto load_b = [&](int s, uint4(&w)[2], u32x2_t(&sc)[2]) {
      // plain loads: the other half of each 128-byte line is requested one
      // step later and should still be in the L2
      w[0] = load16_g(gq + (woff + 64u * s));
      w[1] = load16_g(uq + (woff + 64u * s));
      sc[0] = *reinterpret_cast<gu2_t *>(gsc + (soff + 8u * s));
      sc[1] = *reinterpret_cast<gu2_t *>(usc + (soff + 8u * s));
    };

    f32x4_t acc[2][4];
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) acc[q][mt] = zero4;
    uint4 av[2][2];     // A rows of the next two steps, slot s & 1
    uint4 bw[4][2];     // weight chunks, slot s & 3
    u32x2_t bs[4][2];   // their block scales
    // B(0), A(0), B(1): once A(0) has arrived, B(0) has too (the counter of
    // outstanding loads drains in order) and only B(1) is pending, as at the
    // top of every later pair of steps
    load_b(0, bw[0], bs[0]);
    load_a(0, av[0]);
    load_b(1, bw[1], bs[1]);
    load_b(2, bw[2], bs[2]);
    load_b(3, bw[3], bs[3]);
    load_a(1, av[1]);
    store_a(0, av[0]);
    lds_barrier();
    with_msub((rows + 15) >> 4, [&](auto msc) __attribute__((always_inline)) {
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
#pragma unroll
        for (int q = 0; q < 2; ++q) xpose4(bw[sl][q]);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          // block 4 s + p: both weight tiles' operands (scaled, fp16), then
          // each 16-row tile of A against both
          u32x4_t B[2];
#pragma unroll
          for (int q = 0; q < 2; ++q)
            B[q] = dequant_f16_pairs(word(bw[sl][q], p), scale_pair(bs[sl][q].x, bs[sl][q].y, p));
          uint4 Av[MS];
#pragma unroll
          for (int mt = 0; mt < MS; ++mt) Av[mt] = as[sl & 1][16 * mt + n][4 * p + g];
#pragma unroll
          for (int mt = 0; mt < MS; ++mt) {
            const u32x4_t A = {Av[mt].x, Av[mt].y, Av[mt].z, Av[mt].w};
#pragma unroll
            for (int q = 0; q < 2; ++q) acc[q][mt] = mfma_f16(A, B[q], acc[q][mt]);
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
    // SwiGLU into LDS (the A buffers are free now): lane (n, g) holds rows
    // 16 mt + 4 g + i of column col; rows [64][hi 128 + 8 pad | lo 128 + 8].
    // Rows past the tile's end hold finite values that are never stored.
    uint16_t *st = reinterpret_cast<uint16_t *>(&as[0][0][0]);
    constexpr int kStPlane = 136, kStRow = 2 * kStPlane;
    static_assert(kPfRows * kStRow * 2 <= sizeof(as), "SwiGLU staging must fit the A buffers");
    const int cl = act_pos<MOE_W_INT4_B32>(16 * wave + n);  // tiles start at multiples of 8
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; i += 2) {
        // rows r and r + 1 converted in pairs
        const int r = 16 * mt + 4 * g + i;
        float v[2];
#pragma unroll
        for (int d = 0; d < 2; ++d) {
          const float gv = acc[0][mt][i + d], uv = acc[1][mt][i + d];
          v[d] = gv * __builtin_amdgcn_rcpf(1.f + __expf(-gv)) * uv;
        }
        const uint32_t hi = f32x2_to_bf16x2_rne(v[0], v[1]);
        const uint32_t lo = f32x2_to_bf16x2_rne(v[0] - bf16_lo(hi), v[1] - bf16_hi(hi));
        st[r * kStRow + cl] = static_cast<uint16_t>(hi);
        st[(r + 1) * kStRow + cl] = static_cast<uint16_t>(hi >> 16);
        st[r * kStRow + kStPlane + cl] = static_cast<uint16_t>(lo);
        st[(r + 1) * kStRow + kStPlane + cl] = static_cast<uint16_t>(lo >> 16);
      }
    lds_barrier();
    // 16-byte stores of whole row segments: piece (row, plane, 16 of them)
#pragma unroll
    for (int k2 = 0; k2 < 4; ++k2) {
      const int idx = tid + kGmThreads * k2;
      const int r = idx >> 5, plane = (idx >> 4) & 1, pcs = idx & 15;
      if (r < rows) {
        const uint4 v = *reinterpret_cast<const uint4 *>(st + r * kStRow + plane * kStPlane + 8 * pcs);
        const int rr = m0 + r;
        const size_t off = shared ? static_cast<size_t>(a.n_rows) * a.F + static_cast<size_t>(rr) * a.Fs
                                  : static_cast<size_t>(un.r0 + rr) * a.F;
        uint16_t *arow = reinterpret_cast<uint16_t *>(a.act + off);
        *reinterpret_cast<uint4 *>(arow + plane * F + ct * 128 + 8 * pcs) = v;
      }
    }
    lds_barrier();  // the next item's first A tile reuses the buffers
  }
}

template <int KS>
__global__ void __launch_bounds__(kGmThreads, 4) down_gemm_kernel(FfnArgs a) {
  static_assert(KS % 2 == 0, "the k loop runs over pairs of steps");
  __shared__ uint4 as[2][2][kPfRows][17];  // [buffer][hi, lo plane] act rows in fp16, one k-step
  __shared__ GmUnits units;
  __shared__ int scratch[kGmThreads / 64];
  constexpr int nblk = 4 * KS;  // 32-element blocks per weight row
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int n = lane & 15, g = lane >> 4;
  const int H = a.H;
  const int n_units = gm_units(a, units, scratch);
  const int col_tiles = H / 256;
  const int n_items = units.pre[n_units] * col_tiles;
  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
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
    const int F = shared ? a.Fs : a.F;  // == 128 KS
    // output columns of this lane: hbase + 16 q; 32-bit offsets from
    // block-uniform bases
    const int hbase = ct * 256 + 32 * wave + n;
    const uint32_t row0 = static_cast<uint32_t>((shared ? 0 : un.e) * H + hbase);
    gchar_t *dq = uniform_gptr(shared ? a.sdq : a.dq);
    gchar_t *dsc = uniform_gptr(shared ? a.sds : a.ds);
    uint32_t woff = row0 * (nblk * 16) + 16 * g, soff = row0 * (nblk * 2);
    constexpr uint32_t kW16 = 16 * nblk * 16, kS16 = 16 * nblk * 2;  // 16 rows further

    // A staging: thread t owns piece t % 16 of rows t / 16 + 32 i, both
    // planes (byte offsets of the rows inside the act buffer); rows past
    // the tile's end read its first row (results never stored)
    gchar_t *ag = uniform_gptr(a.act);
    uint32_t aoff[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = (tid >> 4) + 32 * i;
      const int rr = m0 + (r < rows ? r : 0);
      const uint32_t off = shared ? static_cast<uint32_t>(a.n_rows * a.F + rr * a.Fs)
                                  : static_cast<uint32_t>((un.r0 + rr) * a.F);
      aoff[i] = 4 * off + 16 * pc;
    }
    auto load_a = [&](int s, uint4(&v)[4]) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        v[i] = load16_g(ag + (aoff[i] + 256u * s));
        v[2 + i] = load16_g(ag + (aoff[i] + 2u * F + 256u * s));
      }
    };
    auto f16x8 = [](const uint4 &v) {
      return make_uint4(bf16x2_to_f16x2(v.x), bf16x2_to_f16x2(v.y), bf16x2_to_f16x2(v.z), bf16x2_to_f16x2(v.w));
    };
    auto store_a = [&](int buf, const uint4(&v)[4]) {
      // both planes in fp16
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        as[buf][0][(tid >> 4) + 32 * i][pc] = f16x8(v[i]);
        as[buf][1][(tid >> 4) + 32 * i][pc] = f16x8(v[2 + i]);
      }
    };
    auto load_b = [&](int s, uint4(&w)[2], u32x2_t(&sc)[2]) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        w[q] = load16_g(dq + (woff + q * kW16 + 64u * s));
        sc[q] = *reinterpret_cast<gu2_t *>(dsc + (soff + q * kS16 + 8u * s));
      }
    };

    f32x4_t acc[2][4];
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) acc[q][mt] = zero4;
    uint4 av[4];
    uint4 bw[2][2];
    u32x2_t bs[2][2];
    // B(0), A(0), B(1): once A(0) has arrived, B(0) has too (the counter of
    // outstanding loads drains in order) and only B(1) is pending, as at the
    // top of every later pair of steps
    load_b(0, bw[0], bs[0]);
    load_a(0, av);
    load_b(1, bw[1], bs[1]);
    store_a(0, av);
    lds_barrier();
    with_msub((rows + 15) >> 4, [&](auto msc) __attribute__((always_inline)) {
      constexpr int MS = decltype(msc)::value;
      auto step = [&](int s, auto slc) __attribute__((always_inline)) {
        constexpr int sl = decltype(slc)::value;
        pin_u32(woff);
        pin_u32(soff);
#pragma unroll
        for (int i = 0; i < 2; ++i) pin_u32(aoff[i]);
        load_a(min(s + 1, KS - 1), av);  // A(s) is in LDS already; clamped
#pragma unroll
        for (int q = 0; q < 2; ++q) xpose4(bw[sl][q]);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          u32x4_t B[2];
#pragma unroll
          for (int q = 0; q < 2; ++q)
            B[q] = dequant_f16_pairs(word(bw[sl][q], p), scale_pair(bs[sl][q].x, bs[sl][q].y, p));
#pragma unroll
          for (int mt = 0; mt < MS; ++mt) {
            const uint4 vh = as[sl][0][16 * mt + n][4 * p + g];
            const uint4 vl = as[sl][1][16 * mt + n][4 * p + g];
            const u32x4_t Ah = {vh.x, vh.y, vh.z, vh.w}, Al = {vl.x, vl.y, vl.z, vl.w};
#pragma unroll
            for (int q = 0; q < 2; ++q) acc[q][mt] = mfma_f16(Al, B[q], mfma_f16(Ah, B[q], acc[q][mt]));
          }
        }
        load_b(min(s + 2, KS - 1), bw[sl], bs[sl]);
        __builtin_amdgcn_sched_barrier(0);
        store_a(sl ^ 1, av);  // unconditional: no branch inside the step
        lds_barrier();
      };
      for (int s = 0; s < KS; s += 2) {
        step(s, IntC<0>{});
        step(s + 1, IntC<1>{});
      }
    });
    // the tile into LDS (the A buffers are free now), rows of 256 + 4 floats,
    // then 16-byte stores of whole row segments with the row's weight
    float *st = reinterpret_cast<float *>(&as[0][0][0][0]);
    constexpr int kStRow = 260;
    static_assert(kPfRows * kStRow * 4 <= sizeof(as), "output staging must fit the A buffers");
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int c = 32 * wave + 16 * q + n;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) st[(16 * mt + 4 * g + i) * kStRow + c] = acc[q][mt][i];
    }
    lds_barrier();
#pragma unroll
    for (int k2 = 0; k2 < 8; ++k2) {
      const int idx = tid + kGmThreads * k2;
      const int r = idx >> 6, pcs = idx & 63;
      if (r < rows) {
        const float4 v = *reinterpret_cast<const float4 *>(st + r * kStRow + 4 * pcs);
        const int rr = m0 + r;
        const int row = un.r0 + rr;
        const float wgt = shared || !a.row_w ? 1.f : a.row_w[row];
        const size_t orow = shared ? static_cast<size_t>(a.n_rows) + rr : static_cast<size_t>(row);
        *reinterpret_cast<float4 *>(a.rows_out + orow * H + ct * 256 + 4 * pcs) =
            make_float4(v.x * wgt, v.y * wgt, v.z * wgt, v.w * wgt);
      }
    }
    lds_barrier();
  }
}

// ----------------------------------------------------------------- launches

bool prefill_ok(const FfnArgs &a) {
  const int units = (a.Fs > 0 ? 1 : 0) + (a.offsets ? a.max_units : 1);
  return a.fmt == MOE_W_INT4_B32 && a.T > kFusedTokens && (a.Fs == 0 || a.Fs == a.F) && a.H % 128 == 0 &&
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

hipError_t launch_gateup_prefill(const FfnArgs &a, hipStream_t s) {
  if (a.H == 128 * 16 && a.F % 128 == 0 && gm_units_fit(a)) {
    return launch_kernel(gateup_gemm_kernel<16>, dim3(gm_grid(pf_tiles_upper(a) * (a.F / 128), 1)), dim3(kGmThreads), 0,
                         s, a);
  }
  return launch_kernel(gateup_prefill_kernel, dim3(pf_grid(pf_tiles_upper(a) * (a.F / kPfCols))), dim3(kPfThreads), 0,
                       s, a);
}

hipError_t launch_down_prefill(const FfnArgs &a, hipStream_t s) {
  if (a.F == 128 * 4 && a.H % 256 == 0 && gm_units_fit(a)) {
    return launch_kernel(down_gemm_kernel<4>, dim3(gm_grid(pf_tiles_upper(a) * (a.H / 256), 2)), dim3(kGmThreads), 0, s,
                         a);
  }
  return launch_kernel(down_prefill_kernel, dim3(pf_grid(pf_tiles_upper(a) * (a.H / kPfCols))), dim3(kPfThreads), 0,
                       s, a);
}

}  // namespace moe
