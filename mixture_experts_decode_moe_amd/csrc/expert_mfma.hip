// Expert FFN on the bf16 matrix cores, decode batches (int4 and int8).
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
// int8 weights (q stored as a two's-complement byte, fp32 scale per row):
// q itself is exact in bfloat16 (|q| <= 127; converted through fp32), the
// 16x16x16 MFMA takes four consecutive k per lane, the sums run over the
// whole row in the MFMA accumulator with no correction, and the row scale is
// applied once at the end.  The operands keep their natural element order.
//
// Operand layout (v_mfma_f32_16x16x32_bf16, wave64): lane l supplies A row
// l % 16 and B column l % 16, k-group l / 16 (8 consecutive k of the 32);
// the result element (m, n) lands in lane 16 * (m / 4) + n, register m % 4.
// (The 16x16x16 form is the same with 4 k per lane.)  A lane's 16-byte
// weight load covers one whole k-block of one row (32 int4 or 16 int8
// weights); four such loads (k-groups g = 0..3 of four consecutive blocks) are
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

#include "mfma_common.h"
#include "route_common.h"

namespace moe {

// Units of the MFMA kernels: the shared expert's tiles first, then the
// routed units' tiles.
struct MUnit {
  const void *gq, *gs, *uq, *us, *dq, *ds;
  int F, e, r0, n, tile;
  bool shared;
};

// rec (with use_rec): the unit's (expert, first row, rows) record from the
// routing's unit table, read by the caller already; else it is looked up
MOE_DEV bool mfma_unit(const FfnArgs &a, int item, int tiles_r, int tiles_s, int U, MUnit &u, bool use_rec,
                       int4 rec) {
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
  if (use_rec) {
    u.e = rec.x;
    u.r0 = rec.y;
    u.n = rec.z;
  } else if (a.offsets) {
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
// Persistent: one block of KS waves per compute unit; block b takes items
// b, b + G, b + 2G, ...  The T (<= 16) token rows of x are staged in LDS
// once per block, in operand order.  Item: (unit, 8 SwiGLU columns
// f0..f0+7) as one 16-column MFMA tile: columns 0-7 are the gate rows
// f0..f0+7, columns 8-15 the matching up rows.  Wave w multiplies
// block-quads [w JW, w JW + JW) of the hidden dimension; the partial tiles
// are added in LDS in wave order.  The block's items (unit, rows, tokens)
// are looked up once into an LDS table, and each item's weights are
// requested while the previous item is computed and reduced.
constexpr int kGuTable = 128;  // most items one block takes
constexpr int kGuGroup = 4;    // items reduced together

template <int FMT, int JW>
struct GuWeights {
  uint4 w[JW];
  uint32_t s[JW][2];  // int4: the fp16 scales of the four blocks
  float rs;           // int8: the row scale
};

// Base pointers of the routed and shared gate/up weights, read once per
// block into scalar registers.
struct GuPtrs {
  gchar_t *gq, *uq, *gs, *us;      // routed
  gchar_t *sgq, *suq, *sgs, *sus;  // shared
};

MOE_DEV GuPtrs gu_ptrs(const FfnArgs &a) {
  GuPtrs p;
  p.gq = uniform_gptr(a.gq);
  p.uq = uniform_gptr(a.uq);
  p.gs = uniform_gptr(a.gs);
  p.us = uniform_gptr(a.us);
  p.sgq = uniform_gptr(a.sgq);
  p.suq = uniform_gptr(a.suq);
  p.sgs = uniform_gptr(a.sgs);
  p.sus = uniform_gptr(a.sus);
  return p;
}

// This lane's weight and scale bases and its fixed byte offsets, set once
// per block: lanes n < 8 read gate rows, lanes n >= 8 up rows; the routed
// and the shared expert's matrices.  Offsets from these bases fit 32 bits
// (mfma_decode_ok checks the matrix sizes).
struct GuLane {
  gchar_t *q_r, *q_s, *s_r, *s_s;  // weights / scales, routed and shared
  uint32_t w_off;                  // this lane's bytes within a row: 64 (wave JW) + 16 g
  uint32_t n7;                     // the lane's row within the item's gate or up rows
};

template <int FMT, int JW>
MOE_DEV GuLane gu_lane(const GuPtrs &P, int wave, int n, int g) {
  const bool up = n >= 8;
  GuLane L;
  L.q_r = up ? P.uq : P.gq;
  L.q_s = up ? P.suq : P.sgq;
  L.s_r = up ? P.us : P.gs;
  L.s_s = up ? P.sus : P.sgs;
  L.w_off = 64u * static_cast<uint32_t>(wave * JW) + 16u * static_cast<uint32_t>(g);
  L.n7 = static_cast<uint32_t>(n & 7);
  return L;
}

// Loads this lane's part of item (e, f0) (e < 0: the shared expert); e and
// f0 are wave-uniform.  Row f0 + n7 of the gate or up matrix: JW 16-byte
// chunks at w_off + 64 jj, and the chunks' block scales (int4) or the row
// scale (int8).
template <int FMT, int JW, bool SCALES = true>
MOE_DEV void gu_load(const FfnArgs &a, const GuLane &L, int e, int f0, GuWeights<FMT, JW> &w) {
  using Fm = MfmaFmt<FMT>;
  const bool shared = e < 0;
  const uint32_t F = static_cast<uint32_t>(shared ? a.Fs : a.F);
  const uint32_t nblk = static_cast<uint32_t>(a.H / Fm::kBlockK);
  const uint32_t row = (shared ? 0u : static_cast<uint32_t>(e)) * F + static_cast<uint32_t>(f0) + L.n7;
  gchar_t *q = shared ? L.q_s : L.q_r;
  gchar_t *sc = shared ? L.s_s : L.s_r;
  const uint32_t woff = row * (nblk * 16u) + L.w_off;
#pragma unroll
  for (int jj = 0; jj < JW; ++jj) w.w[jj] = load_stream16_g(q + (woff + 64u * jj));
  if constexpr (FMT == MOE_W_INT4_B32 && !SCALES) {
    w.rs = 1.f;  // the block scales come from LDS (gateup_mfma_kernel with SCL)
  } else if constexpr (FMT == MOE_W_INT4_B32) {
    // the four fp16 scales of each chunk: 8 bytes at 8 (wave JW + jj)
    const uint32_t soff = row * (nblk * 2u) + (L.w_off & ~63u) / 8u;
#pragma unroll
    for (int jj = 0; jj < JW; ++jj) {
      const u32x2_t sv = *reinterpret_cast<gu2_t *>(sc + (soff + 8u * jj));
      w.s[jj][0] = sv.x;
      w.s[jj][1] = sv.y;
    }
    w.rs = 1.f;
  } else {
    w.rs = *reinterpret_cast<gf32_t *>(sc + row * 4u);
  }
}

// Unit of item i: e (-1 for the shared expert), first row, rows, f0.
MOE_DEV void gu_item(const FfnArgs &a, int i, int tiles_r, int tiles_s, int &e, int &r0, int &n, int &f0) {
  if (i < tiles_s) {
    e = -1;
    r0 = 0;
    n = a.T;
    f0 = i * 8;
    return;
  }
  const int k = (i - tiles_s) / tiles_r;
  f0 = (i - tiles_s - k * tiles_r) * 8;
  if (a.offsets) {
    e = a.active[k];
    r0 = a.offsets[e];
    n = a.offsets[e + 1] - r0;
  } else {
    e = 0;
    r0 = 0;
    n = a.n_rows;
  }
}

// SCL: the scales of a chunk's items are staged in LDS by direct loads,
// instead of every wave requesting a few bytes of each of its items' 16
// scale rows (which doubled the requests of the weight stream for an eighth
// of its bytes).  int4 only (H = 2048, 16 waves, 8 items a chunk): wave w
// loads the 128-byte block-scale rows of the gate or up half of item w / 2.
// (The int8 row scales, one float a row, staged the same way by one wave
// made that kernel slower: they are a sixty-fourth of its bytes.)
template <int FMT, int JW, int NI, bool SCL>
__global__ void __launch_bounds__(1024) gateup_mfma_kernel(FfnArgs a) {
  using Fm = MfmaFmt<FMT>;
  using Vec = typename Fm::Vec;
  constexpr bool kInt4 = FMT == MOE_W_INT4_B32;
  extern __shared__ uint4 xs_lds[];  // [T][H/8 + 1] 16-byte pieces of x
  __shared__ f32x4_t red[kGuGroup][kGuMaxWaves][64];  // partial tiles of a group of items
  __shared__ __attribute__((aligned(16))) int tab[kGuTable][4];  // e, r0, n (<= 16), f0
  __shared__ int toks[kGuTable][16];
  __shared__ uint32_t act_st[NI][16][8];  // SwiGLU outputs of a chunk: bf16 hi | lo << 16
  // SCL: item i's 16 scale rows of 8 pieces (16 bytes, 8 blocks each), the
  // piece p of row r at slot p ^ (r & 7)
  __shared__ uint4 sc_lds[SCL ? NI * 128 : 1];
  static_assert(!SCL || (kInt4 && JW == 1 && NI == 8), "SCL: int4, H = 2048, 8 items a chunk");
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int KS = blockDim.x >> 6;
  const int n = lane & 15;
  const int g = lane >> 4;
  const int H = a.H, T = a.T;
  const int pieces = H / 8;  // 16-byte pieces per x row
  const int xstride = pieces + 1;
  const Vec cvec = Fm::corr();
  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
  // the in-kernel routing's LDS shares the partial-tile buffer
  RouteLds &L = *reinterpret_cast<RouteLds *>(&red[0][0][0]);
  static_assert(sizeof(RouteLds) <= sizeof(red), "routing LDS must fit the partial-tile buffer");

  auto stage_x = [&](int t0, int nthr) {  // threads t0.. stage the x rows in LDS
    for (int base = tid - t0; base < T * pieces; base += nthr * kStageBatch) {
      uint4 v[kStageBatch];
#pragma unroll
      for (int b = 0; b < kStageBatch; ++b) {
        const int i = base + b * nthr;
        v[b] = i < T * pieces ? reinterpret_cast<const uint4 *>(a.x)[i] : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int b = 0; b < kStageBatch; ++b) {
        const int i = base + b * nthr;
        if (i < T * pieces) {
          const int t = i / pieces, k = i - t * pieces;
          uint4 o = v[b];
          if constexpr (kInt4) {
            const u32x4_t pp = pair_permute(v[b]);
            o = make_uint4(pp.x, pp.y, pp.z, pp.w);
          }
          xs_lds[t * xstride + k] = o;
        }
      }
    }
  };

  int U;
  uint4 xv[4];  // route_here: the first x pieces, requested before the routing
  if (a.route_here) {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int i = tid + b * blockDim.x;
      xv[b] = i < T * pieces ? reinterpret_cast<const uint4 *>(a.x)[i] : make_uint4(0, 0, 0, 0);
    }
    // the x rows go to LDS while the partial logits are in flight
    auto stage_xv = [&]() {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int i = tid + b * blockDim.x;
        if (i < T * pieces) {
          const int t = i / pieces, k = i - t * pieces;
          uint4 o = xv[b];
          if constexpr (kInt4) {
            const u32x4_t pp = pair_permute(xv[b]);
            o = make_uint4(pp.x, pp.y, pp.z, pp.w);
          }
          xs_lds[t * xstride + k] = o;
        }
      }
    };
    // every block routes the batch (the last block, which has the fewest
    // items, also publishes it)
    const int npl = (a.route.E + 63) / 64;
    if (npl <= 1)
      route_in_block_small<1>(a.route, L, blockIdx.x == gridDim.x - 1, stage_xv);
    else if (npl <= 2)
      route_in_block_small<2>(a.route, L, blockIdx.x == gridDim.x - 1, stage_xv);
    else
      route_in_block_small<4>(a.route, L, blockIdx.x == gridDim.x - 1, stage_xv);  // E <= 256 on this path
    U = L.n_active;
  } else {
    U = routed_units(a);
  }
  const int tiles_r = a.F / 8, tiles_s = a.Fs / 8;
  const int n_items = tiles_s + U * tiles_r;
  // block b owns the contiguous items [b C, b C + C) (C <= kGuTable)
  const int C = (n_items + gridDim.x - 1) / gridDim.x;
  const int first = blockIdx.x * C;
  const int my_items = n_items > first ? min(C, n_items - first) : 0;
  if (my_items == 0) return;

  if (a.route_here) {
    // the item table from the routing in LDS, then the x rows
    if (tid < my_items) {
      const int i = first + tid;
      int e, r0, nn, f0;
      if (i < tiles_s) {
        e = -1;
        r0 = 0;
        nn = T;
        f0 = i * 8;
      } else {
        const int k = (i - tiles_s) / tiles_r;
        f0 = (i - tiles_s - k * tiles_r) * 8;
        e = L.active[k];
        r0 = L.off[e];
        nn = L.cnt[e];
      }
      nn = nn > 16 ? 16 : nn;
      tab[tid][0] = e;
      tab[tid][1] = r0;
      tab[tid][2] = nn;
      tab[tid][3] = f0;
#pragma unroll
      for (int m = 0; m < 16; ++m) toks[tid][m] = m < nn ? (e < 0 ? m : L.row_tok[r0 + m]) : 0;
    }
    if (T * pieces > 4 * static_cast<int>(blockDim.x)) {  // the rest of the rows
      for (int base = tid + 4 * blockDim.x; base < T * pieces; base += blockDim.x) {
        const int t = base / pieces, k = base - t * pieces;
        uint4 o = reinterpret_cast<const uint4 *>(a.x)[base];
        if constexpr (kInt4) {
          const u32x4_t pp = pair_permute(o);
          o = make_uint4(pp.x, pp.y, pp.z, pp.w);
        }
        xs_lds[t * xstride + k] = o;
      }
    }
  } else if (tid < kGuTable) {
    // waves 0-1 look up the block's items (unit, rows, tokens; one thread per
    // item, all in parallel) while the other waves stage the x rows in LDS
    if (tid < my_items) {
      int e, r0, nn, f0;
      gu_item(a, first + tid, tiles_r, tiles_s, e, r0, nn, f0);
      nn = nn < 0 ? 0 : (nn > 16 ? 16 : nn);  // one 16-row tile (T <= 16)
      tab[tid][0] = e;
      tab[tid][1] = r0;
      tab[tid][2] = nn;
      tab[tid][3] = f0;
      int tk[16];
      const int last = a.n_rows > 0 ? a.n_rows - 1 : 0;
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        // unconditional (clamped) loads, selected afterwards
        const int ri = min(r0 + m, last);
        const int raw = a.row_tok ? a.row_tok[ri] : ri;
        const int t = m < nn ? (e < 0 ? m : raw) : 0;
        tk[m] = t < 0 ? 0 : (t >= T ? T - 1 : t);  // memory safety for malformed row lists
      }
#pragma unroll
      for (int m = 0; m < 16; ++m) toks[tid][m] = tk[m];
    }
  } else {
    stage_x(kGuTable, blockDim.x - kGuTable);
  }
  lds_barrier();

  // Chunks of NI items as straight-line code: every weight load of a chunk
  // is issued first (unconditionally: a missing item re-requests the
  // chunk's first item, already in flight), so the wait before each item
  // leaves the later items' loads in flight.
  const GuLane GL = gu_lane<FMT, JW>(gu_ptrs(a), wave, n, g);
  // the unit of the last item multiplied, its x row pointer and correction
  // products (wave-uniform unit; kept across chunks)
  constexpr bool kKeepCorr = kInt4 && JW == 1;
  int run_e = -2;  // no unit (-1 is the shared expert)
  const uint16_t *xrow = nullptr;
  f32x4_t run_corr[kKeepCorr ? 4 : 1];
  for (int c0 = 0; c0 < my_items; c0 += NI) {
    GuWeights<FMT, JW> w[NI];
    // the chunk's item records first (one LDS read each, all in flight
    // together), made wave-uniform, then every weight request
    int te[NI], tf[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int it = c0 + i < my_items ? c0 + i : c0;
      const int4 rec = *reinterpret_cast<const int4 *>(tab[it]);
      te[i] = rec.x;
      tf[i] = rec.w;
    }
    if constexpr (SCL) {
      // wave w: scale rows 8 (w & 1) .. + 7 (gate: 0-7, up: 8-15) of item w / 2
      // of the chunk, one 1 KB direct load; lane l row l / 8, piece
      // (l % 8) ^ (row % 8) into slot l % 8
      const int hi = wave >> 1, half = wave & 1;
      const int it = c0 + hi < my_items ? c0 + hi : c0;
      const int e = __builtin_amdgcn_readfirstlane(tab[it][0]);
      const int f0 = __builtin_amdgcn_readfirstlane(tab[it][3]);
      const bool shared = e < 0;
      const uint32_t F = static_cast<uint32_t>(shared ? a.Fs : a.F);
      const int r = lane >> 3;
      const uint32_t row = (shared ? 0u : static_cast<uint32_t>(e)) * F + static_cast<uint32_t>(f0) + r;
      gchar_t *sb = half ? (shared ? uniform_gptr(a.sus) : uniform_gptr(a.us))
                         : (shared ? uniform_gptr(a.sgs) : uniform_gptr(a.gs));
      __builtin_amdgcn_global_load_lds(sb + (row * 128u + 16u * static_cast<uint32_t>((lane & 7) ^ (r & 7))),
                                       (__attribute__((address_space(3))) void *)(sc_lds + hi * 128 + half * 64),
                                       16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < NI; ++i)
      gu_load<FMT, JW, !SCL>(a, GL, __builtin_amdgcn_readfirstlane(te[i]), __builtin_amdgcn_readfirstlane(tf[i]),
                             w[i]);
    if constexpr (SCL) {
      // a wave's scale load is older than its NI JW weight loads; once every
      // wave's has landed the chunk's scales are in LDS
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(NI * JW));
      lds_barrier();
    }
    // groups of kGuGroup items: every wave's partial tiles of the group go to
    // LDS, then one pass adds them and applies SwiGLU (two barriers a group)
#pragma unroll
    for (int g0 = 0; g0 < NI; g0 += kGuGroup) {
#pragma unroll
      for (int j = 0; j < kGuGroup; ++j) {
        const int i = g0 + j;
        const int it = c0 + i;
        if (i < NI && it < my_items) {
#pragma unroll
          for (int jj = 0; jj < JW; ++jj) xpose4(w[i].w[jj]);
          if constexpr (SCL) {
            // the scales of blocks 4 q .. 4 q + 3 of row n: half q % 2 of piece q / 2
#pragma unroll
            for (int jj = 0; jj < JW; ++jj) {
              const int q = wave * JW + jj;
              const uint2 sv =
                  reinterpret_cast<const uint2 *>(sc_lds + i * 128 + n * 8 + ((q >> 1) ^ (n & 7)))[q & 1];
              w[i].s[jj][0] = sv.x;
              w[i].s[jj][1] = sv.y;
            }
          }
          // Slots m >= nrows read token 0's row (a finite operand): their
          // output rows are never read, and MFMA rows do not mix.  Items of
          // one unit share their token rows, so the row pointer and (int4,
          // one block-quad a wave) the correction products are formed once
          // per run of items of the same unit.
          const int e_i = __builtin_amdgcn_readfirstlane(te[i]);
          if (e_i != run_e) {
            run_e = e_i;
            xrow = reinterpret_cast<const uint16_t *>(xs_lds + toks[it][n] * xstride);
            if constexpr (kKeepCorr) {
#pragma unroll
              for (int p = 0; p < 4; ++p) run_corr[p] = Fm::mfma(Fm::a_plane(xrow, 4 * wave + p, g), cvec, zero4);
            }
          }
          f32x4_t acc = zero4;
#pragma unroll
          for (int jj = 0; jj < JW; ++jj)
#pragma unroll
            for (int p = 0; p < 4; ++p) {
              // staged x is already in operand order
              const Vec xa = Fm::a_plane(xrow, 4 * (wave * JW + jj) + p, g);
              if constexpr (kInt4) {
                // per block: -136 * sum(x) as the accumulator input, then the scale
                const f32x4_t c0v = kKeepCorr ? run_corr[p] : Fm::mfma(xa, cvec, zero4);
                const f32x4_t c = Fm::mfma(xa, Fm::b_w(word(w[i].w[jj], p)), c0v);
                acc = fma4(scale4(w[i].s[jj][0], w[i].s[jj][1], p), c, acc);
              } else {
                acc = Fm::mfma(xa, Fm::b_w(word(w[i].w[jj], p)), acc);
              }
            }
          if constexpr (!kInt4) acc = acc * w[i].rs;
          red[j][wave][lane] = acc;
        }
      }
      lds_barrier();
      // thread (j, m, f): token row m of item g0 + j, gate and up columns
      // f0 + f and their 8 + f partner, added in wave order
      if (tid < kGuGroup * 128) {
        const int j = tid >> 7, m = (tid >> 3) & 15, f = tid & 7;
        const int i = g0 + j, it = c0 + i;
        if (i < NI && it < my_items && m < tab[it][2]) {
          const int src = 16 * (m >> 2) + f, r = m & 3;
          float gv = 0.f, uv = 0.f;
          for (int ww = 0; ww < KS; ++ww) {
            gv += red[j][ww][src][r];
            uv += red[j][ww][src + 8][r];
          }
          const float v = gv / (1.f + expf(-gv)) * uv;
          const uint16_t hi = f32_to_bf16_rne(v);
          const uint16_t lo = f32_to_bf16_rne(v - bf16_to_f32(hi));
          act_st[i][m][f] = static_cast<uint32_t>(hi) | (static_cast<uint32_t>(lo) << 16);
        }
      }
      lds_barrier();
    }
    // the chunk's SwiGLU rows to global memory: thread (i, m, f)
    if (tid < NI * 128) {
      const int i = tid >> 7, m = (tid >> 3) & 15, f = tid & 7;
      const int it = c0 + i;
      if (it < my_items && m < tab[it][2]) {
        const int e = tab[it][0], r0 = tab[it][1], f0 = tab[it][3];
        const int F = e < 0 ? a.Fs : a.F;
        const size_t off = e < 0 ? static_cast<size_t>(a.n_rows) * a.F + static_cast<size_t>(m) * a.Fs
                                 : static_cast<size_t>(r0 + m) * a.F;
        uint16_t *arow = reinterpret_cast<uint16_t *>(a.act + off);
        const uint32_t v = act_st[i][m][f];
        const int pos = act_pos<FMT>(f0 + f);
        arow[pos] = static_cast<uint16_t>(v & 0xFFFFu);
        arow[F + pos] = static_cast<uint16_t>(v >> 16);
      }
    }
    lds_barrier();
  }
}

// --------------------------------------------------------------------- down
//
// Item: (unit, 64 output rows h0..h0+63 as four 16-row tiles).  Wave w
// multiplies block-quads [w JW, w JW + JW) of the SwiGLU dimension.  The
// routing weight is applied when the summed tile is stored.
template <int FMT, int JW>
__global__ void __launch_bounds__(512) down_mfma_kernel(FfnArgs a) {
  using Fm = MfmaFmt<FMT>;
  using Vec = typename Fm::Vec;
  constexpr bool kInt4 = FMT == MOE_W_INT4_B32;
  __shared__ f32x4_t red[kDnMaxWaves][4][64];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int KS = blockDim.x >> 6;
  const int n = lane & 15;
  const int g = lane >> 4;
  const int H = a.H;
  const int tiles = H / 64;
  const int tiles_s = a.Fs > 0 ? tiles : 0;
  // With the routing's unit table, the first item's record is requested
  // together with the unit count (one round trip instead of three
  // dependent reads: count, active list, offsets).
  int4 rec0 = make_int4(0, 0, 0, 0);
  if (a.units) {
    const int k0 = blockIdx.x >= tiles_s ? (blockIdx.x - tiles_s) / tiles : 0;
    rec0 = reinterpret_cast<const int4 *>(a.units)[min(k0, a.max_units - 1)];
  }
  const int U = routed_units(a);
  const int n_items = tiles_s + U * tiles;
  const Vec cvec = Fm::corr();
  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};

  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    MUnit u;
    int4 rec;
    if (a.units && item != static_cast<int>(blockIdx.x) && item >= tiles_s)
      rec = reinterpret_cast<const int4 *>(a.units)[min((item - tiles_s) / tiles, a.max_units - 1)];
    else
      rec = rec0;
    if (!mfma_unit(a, item, tiles, tiles_s, U, u, a.units != nullptr, rec) || u.n <= 0) continue;
    const int h0 = u.tile * 64;
    const int F = u.F;
    const int nblk = F / Fm::kBlockK;
    const size_t row_bytes = static_cast<size_t>(nblk) * 16;
    uint4 wd[JW][4];
    uint32_t sd[JW][4][2];
    float rs[4] = {1.f, 1.f, 1.f, 1.f};
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const size_t row = static_cast<size_t>(u.e) * H + h0 + 16 * nt + n;
      const uint4 *dp = reinterpret_cast<const uint4 *>(static_cast<const char *>(u.dq) + row * row_bytes);
#pragma unroll
      for (int jj = 0; jj < JW; ++jj) {
        const int j = wave * JW + jj;
        wd[jj][nt] = load_stream16(dp + 4 * j + g);
        if constexpr (kInt4) {
          const uint32_t *sp = reinterpret_cast<const uint32_t *>(static_cast<const uint16_t *>(u.ds) + row * nblk);
          sd[jj][nt][0] = sp[2 * j];
          sd[jj][nt][1] = sp[2 * j + 1];
        }
      }
      if constexpr (!kInt4) rs[nt] = static_cast<const float *>(u.ds)[row];
    }
    // activation rows of the first 16 rows, requested before the weights are
    // waited for
    Vec ah[JW][4], al[JW][4];
    // rows m >= u.n read the unit's first row: their output rows are never
    // stored, and MFMA rows do not mix
    auto load_a = [&](int m0) {
      const int m = m0 + n;
      const uint16_t *hp = reinterpret_cast<const uint16_t *>(a.act + mrow_act(a, u, u.r0 + (m < u.n ? m : 0)));
      const uint16_t *lp = hp + F;  // lo plane follows the hi plane
#pragma unroll
      for (int jj = 0; jj < JW; ++jj)
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int b = 4 * (wave * JW + jj) + p;
          ah[jj][p] = Fm::a_plane(hp, b, g);
          al[jj][p] = Fm::a_plane(lp, b, g);
        }
    };
    // the routing weights of the rows this lane stores (rows m0 + 4 g + i),
    // requested with the act rows rather than after the products
    float rw[4];
    auto load_rw = [&](int m0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int mm = min(m0 + 4 * g + i, u.n - 1);
        rw[i] = u.shared || !a.row_w ? 1.f : a.row_w[u.r0 + mm];
      }
    };
    load_a(0);
    load_rw(0);
#pragma unroll
    for (int jj = 0; jj < JW; ++jj)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) xpose4(wd[jj][nt]);

    for (int m0 = 0; m0 < u.n; m0 += 16) {
      if (m0 > 0) {
        load_a(m0);
        load_rw(m0);
      }
      // the weight words are converted inside the loop (a unit rarely has
      // more than 16 rows; hoisting the conversions would keep sixty-four
      // more registers live and cut the blocks a compute unit holds)
#pragma unroll
      for (int jj = 0; jj < JW; ++jj)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          asm volatile("" : "+v"(wd[jj][nt].x), "+v"(wd[jj][nt].y), "+v"(wd[jj][nt].z), "+v"(wd[jj][nt].w));
          if constexpr (kInt4) asm volatile("" : "+v"(sd[jj][nt][0]), "+v"(sd[jj][nt][1]));
        }
      f32x4_t acc[4] = {zero4, zero4, zero4, zero4};
#pragma unroll
      for (int jj = 0; jj < JW; ++jj)
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          if constexpr (kInt4) {
            f32x4_t c0 = Fm::mfma(ah[jj][p], cvec, zero4);
            c0 = Fm::mfma(al[jj][p], cvec, c0);
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
              const Vec bw = Fm::b_w(word(wd[jj][nt], p));
              f32x4_t c = Fm::mfma(ah[jj][p], bw, c0);
              c = Fm::mfma(al[jj][p], bw, c);
              acc[nt] = fma4(scale4(sd[jj][nt][0], sd[jj][nt][1], p), c, acc[nt]);
            }
          } else {
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
              const Vec bw = Fm::b_w(word(wd[jj][nt], p));
              acc[nt] = Fm::mfma(ah[jj][p], bw, acc[nt]);
              acc[nt] = Fm::mfma(al[jj][p], bw, acc[nt]);
            }
          }
        }
      if constexpr (!kInt4) {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) acc[nt] = acc[nt] * rs[nt];
      }
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) red[wave][nt][lane] = acc[nt];
      lds_barrier();
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
            const int orow = u.shared ? a.n_rows + r : r;
            a.rows_out[static_cast<size_t>(orow) * H + h] = v[i] * rw[i];
          }
        }
      }
      lds_barrier();
    }
  }
}

// ----------------------------------------------------------------- launches

static int mfma_grid(int items) { return items < 1 ? 1 : (items < 4096 ? items : 4096); }

// Block-quads J = K / (4 kBlockK) split over KS waves of JW each, KS a
// power of two in [4, max_waves], JW in {1, 2, 4}.
static bool split_k(int K, int block_k, int max_waves, int &jw, int &ks) {
  const int quad = 4 * block_k;
  const int J = K / quad;
  if (K % quad || J < 4) return false;
  ks = J <= max_waves ? J : max_waves;
  if (ks & (ks - 1)) return false;
  jw = J / ks;
  return jw * ks == J && (jw == 1 || jw == 2 || jw == 4);
}

static int block_k(int fmt) { return fmt == MOE_W_INT4_B32 ? 32 : 16; }

bool mfma_decode_ok(const FfnArgs &a) {
  int jw, ks;
  // staged x plus the gate/up kernel's fixed LDS (partial tiles, item
  // table, SwiGLU staging) must fit one compute unit's 160 KiB
  const size_t lds = static_cast<size_t>(a.T) * (a.H / 8 + 1) * 16 + 80 * 1024;
  // the gate/up kernel holds at most 16 rows of a unit (one MFMA tile):
  // every unit's rows are among the n_rows routed rows, and with distinct
  // experts per token a unit has at most T rows
  const bool rows16 = a.n_rows <= 16 || a.distinct_ids;
  // the gate/up kernel addresses weights and scales with 32-bit offsets
  const uint64_t mat_bytes = static_cast<uint64_t>(a.n_experts > 0 ? a.n_experts : 1) * a.F * a.H;
  const bool off32 = mat_bytes < (1ull << 32) && static_cast<uint64_t>(a.Fs) * a.H < (1ull << 32);
  return a.path != kPathPrefill && rows16 && off32 && (a.fmt == MOE_W_INT4_B32 || a.fmt == MOE_W_INT8_ROW) &&
         a.T <= kFusedTokens && lds <= 160 * 1024 &&
         (a.Fs == 0 || a.Fs == a.F) && split_k(a.H, block_k(a.fmt), kGuMaxWaves, jw, ks) &&
         split_k(a.F, block_k(a.fmt), kDnMaxWaves, jw, ks);
}

// Compute units of the current device (cached per device).
static int cu_count() {
  static int cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    cached[dev] = v;
  }
  return cached[dev];
}

template <int FMT, int JW>
static hipError_t launch_gateup_mfma_t(const FfnArgs &a, int ks, hipStream_t s) {
  // items per chunk: about 128 KiB of weights in flight per block
  constexpr int D = FMT == MOE_W_INT4_B32 ? (JW == 1 ? 8 : 4) : (JW == 1 ? 8 : 4);
  const size_t lds = static_cast<size_t>(a.T) * (a.H / 8 + 1) * 16;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&gateup_mfma_kernel<FMT, JW, D, false>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  // one block per compute unit, at most kGuTable items each (the grid is
  // sized for the largest possible routing; blocks past the last item exit)
  const int items = a.Fs / 8 + a.max_units * (a.F / 8);
  const int cus = cu_count();
  int grid = (items + kGuTable - 1) / kGuTable;
  if (grid < cus) grid = items < cus ? (items < 1 ? 1 : items) : cus;
  if constexpr (FMT == MOE_W_INT4_B32 && JW == 1 && D == 8) {
    if (a.H == 2048 && ks == 16) {
      if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&gateup_mfma_kernel<FMT, JW, D, true>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
        if (e != hipSuccess) return e;
      }
      return launch_kernel(gateup_mfma_kernel<FMT, JW, D, true>, dim3(grid), dim3(64 * ks), lds, s, a.ev, a);
    }
  }
  return launch_kernel(gateup_mfma_kernel<FMT, JW, D, false>, dim3(grid), dim3(64 * ks), lds, s, a.ev, a);
}

template <int FMT>
static hipError_t launch_gateup_mfma_f(const FfnArgs &a, hipStream_t s) {
  int jw, ks;
  split_k(a.H, block_k(FMT), kGuMaxWaves, jw, ks);
  if (jw == 1) return launch_gateup_mfma_t<FMT, 1>(a, ks, s);
  if (jw == 2) return launch_gateup_mfma_t<FMT, 2>(a, ks, s);
  return launch_gateup_mfma_t<FMT, 4>(a, ks, s);
}

template <int FMT>
static hipError_t launch_down_mfma_f(const FfnArgs &a, hipStream_t s) {
  int jw, ks;
  split_k(a.F, block_k(FMT), kDnMaxWaves, jw, ks);
  const int tiles = a.H / 64;
  // blocks loop over items: four a compute unit cover a decode call's items
  // in one round without thousands of blocks that find none
  const int items = (a.Fs > 0 ? tiles : 0) + a.max_units * tiles;
  const int cap = 4 * cu_count();
  const int grid = mfma_grid(items < cap ? items : cap);
  if (jw == 1)
    return launch_kernel(down_mfma_kernel<FMT, 1>, dim3(grid), dim3(64 * ks), 0, s, a.ev, a);
  else if (jw == 2)
    return launch_kernel(down_mfma_kernel<FMT, 2>, dim3(grid), dim3(64 * ks), 0, s, a.ev, a);
  else
    return launch_kernel(down_mfma_kernel<FMT, 4>, dim3(grid), dim3(64 * ks), 0, s, a.ev, a);
}

hipError_t launch_gateup_mfma(const FfnArgs &a, hipStream_t s) {
  return a.fmt == MOE_W_INT4_B32 ? launch_gateup_mfma_f<MOE_W_INT4_B32>(a, s)
                                 : launch_gateup_mfma_f<MOE_W_INT8_ROW>(a, s);
}

hipError_t launch_down_mfma(const FfnArgs &a, hipStream_t s) {
  return a.fmt == MOE_W_INT4_B32 ? launch_down_mfma_f<MOE_W_INT4_B32>(a, s) : launch_down_mfma_f<MOE_W_INT8_ROW>(a, s);
}

}  // namespace moe
