// Down projection fused with the combine, for decode batches of a few
// tokens (whole layer calls only).
//
// The pages end the MoE layer by adding every selected expert's output,
// weighted, plus the shared expert's ("Models and backends", What was
// tuned; "Qwen3.6-35B-A3B: pictures, several requests at once and speed",
// Speed (0.1.45)).  When the batch is a few tokens the down projection and
// that sum fit one launch: a block owns eight output features h0..h0+7 for
// every unit (the shared expert and each active expert), computes each
// unit's rows for those features and adds them per token in slot order, so
// no expert output row goes through global memory and the separate
// combine launch with its chain of dependent reads disappears.
//
// Matrix-core tile.  One 16x16 MFMA tile covers the eight features twice:
// B column n holds feature h0 + (n & 7) over half n >> 3 of the SwiGLU
// dimension, A row m holds token row m & 7 of the unit over half m >> 3.
// Only the tile elements whose row and column halves agree are kept.  A
// unit thus has at most eight rows (T <= 8), and the operands, the exact
// integer products and the per-block scales are those of the decode down
// kernel: bf16 hi + lo parts of the SwiGLU rows, weights as magic bf16 pairs
// (int4: q + 136, -136 sum(x) per block through one more MFMA, fp16 block
// scale in fp32; int8: q itself and the row scale).  Each block-quad of the SwiGLU dimension gives one partial,
// summed from zero over its four blocks exactly as one wave of the down
// kernel sums it; the partials are added in quad order, multiplied by the
// routing weight and summed in slot order as the combine kernel does, so a
// token gets the same bits from this launch as from the two-launch path
// (which a batch of more tokens takes).
//
// Data flow.  The block stages every SwiGLU row of the call (routed and
// shared) in LDS together with the unit table, the slot positions and the
// routing weights (one round of independent reads), then each wave takes
// units w, w + 8, ...: it requests the weights of up to kDcUpw units at
// once, multiplies them against the staged rows and leaves the kept tile
// elements in LDS.  A last pass adds, for every token, each slot's row times
// its routing weight in slot order, then the shared expert's row, and
// writes y (and the residual sum when asked for).
#include <math.h>

#include "mfma_common.h"

namespace moe {

constexpr int kDcMaxThreads = 1024;  // up to 16 waves, one per unit when they fit
constexpr int kDcFeat = 8;           // output features per block
constexpr int kDcUpw = 2;            // units a wave requests at once
constexpr int kDcMaxK = 16;          // slots per token
constexpr int kDcStage = 8;          // 16-byte SwiGLU pieces a thread stages
constexpr size_t kDcLdsBytes = 144 * 1024;  // staged SwiGLU rows and partials

// LDS row stride of a staged SwiGLU row (hi plane, lo plane, 16 bytes of
// padding so consecutive rows start in different banks).
__host__ __device__ inline int dc_row_bytes(int F) { return 4 * F + 16; }

// Weights of one unit for this lane's column: NQ block-quads of its half.
template <int FMT, int NQ>
struct DcWeights {
  uint4 w[NQ];
  uint32_t s[NQ][2];  // int4: fp16 scales of each quad's four blocks
  float rs;           // int8: row scale
};

template <int FMT, int NQ>
__global__ void __launch_bounds__(kDcMaxThreads) down_combine_kernel(DownCombineArgs d) {
  using Fm = MfmaFmt<FMT>;
  using Vec = typename Fm::Vec;
  constexpr bool kInt4 = FMT == MOE_W_INT4_B32;
  constexpr int NBh = 4 * NQ;  // blocks per half row
  extern __shared__ uint4 dc_lds[];
  const FfnArgs &a = d.f;
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int W = nthr >> 6;  // waves
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int n = lane & 15;
  const int g = lane >> 4;
  const int H = a.H, F = a.F, T = a.T, K = d.K;
  const bool has_shared = a.Fs > 0;
  const int n_rows_all = a.n_rows + (has_shared ? T : 0);
  const int rstride = dc_row_bytes(F);
  char *act_l = reinterpret_cast<char *>(dc_lds);
  float *pout = reinterpret_cast<float *>(act_l + static_cast<size_t>(n_rows_all) * rstride);  // [2 NQ][rows][8]
  const int h0 = blockIdx.x * kDcFeat;
  const int nblk = F / Fm::kBlockK;
  const int hb = n >> 3;          // half of this lane's B column
  const int hcol = h0 + (n & 7);  // its output feature
  const int ha = n >> 3;          // half of this lane's A row
  const int ra = n & 7;           // token row of this lane's A row
  const Vec cvec = Fm::corr();
  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
  gchar_t *dq_r = uniform_gptr(a.dq), *ds_r = uniform_gptr(a.ds);
  gchar_t *dq_s = uniform_gptr(a.sdq), *ds_s = uniform_gptr(a.sds);
  const int n_units = min(max(*a.n_active, 0), a.max_units) + (has_shared ? 1 : 0);

  // Unit u: the shared expert first (when present), then the table's units
  // (read straight from global memory: the same address in every lane).
  struct Unit {
    int e, r0, nr;
    bool shared;
  };
  auto unit = [&](int u) {
    Unit un;
    un.shared = has_shared && u == 0;
    const int k = min(max(u - (has_shared ? 1 : 0), 0), a.max_units - 1);
    int4 rec = reinterpret_cast<const int4 *>(d.units)[k];
    // requested unconditionally (not only for routed units)
    asm volatile("" : "+v"(rec.x), "+v"(rec.y), "+v"(rec.z));
    un.e = un.shared ? 0 : min(max(rec.x, 0), d.E - 1);
    un.r0 = un.shared ? a.n_rows : min(max(rec.y, 0), a.n_rows);
    un.nr = un.shared ? T : min(max(rec.z, 0), min(8, a.n_rows - un.r0));
    return un;
  };
  auto load_unit = [&](const Unit &un, DcWeights<FMT, NQ> &w) {
    const size_t row = static_cast<size_t>(un.e) * H + hcol;
    gchar_t *q = (un.shared ? dq_s : dq_r) + row * nblk * 16;
#pragma unroll
    for (int jj = 0; jj < NQ; ++jj) w.w[jj] = load_stream16_g(q + 16 * (4 * (hb * NQ + jj) + g));
    gchar_t *sc = un.shared ? ds_s : ds_r;
    if constexpr (kInt4) {
      gu32_t *sp = reinterpret_cast<gu32_t *>(sc + row * nblk * 2);
#pragma unroll
      for (int jj = 0; jj < NQ; ++jj) {
        const int j = hb * NQ + jj;
        w.s[jj][0] = sp[2 * j];
        w.s[jj][1] = sp[2 * j + 1];
      }
      w.rs = 1.f;
    } else {
      w.rs = reinterpret_cast<gf32_t *>(sc)[row];
    }
  };
  // requests the weights of the wave's units in the chunk starting at c0 (a
  // missing unit re-requests unit 0)
  Unit un[kDcUpw];
  DcWeights<FMT, NQ> w[kDcUpw];
  auto issue = [&](int c0) {
    // every table read first, then every weight request
#pragma unroll
    for (int j = 0; j < kDcUpw; ++j) {
      const int u = c0 + wave + W * j;
      un[j] = unit(u < n_units ? u : 0);
    }
#pragma unroll
    for (int j = 0; j < kDcUpw; ++j) load_unit(un[j], w[j]);
  };
  auto compute = [&](int c0) {
#pragma unroll
    for (int j = 0; j < kDcUpw; ++j) {
      if (c0 + wave + W * j >= n_units) continue;  // wave-uniform
      const int r0 = un[j].r0, nr = un[j].nr;
      const bool mv = ra < nr;
      const char *arow = act_l + static_cast<size_t>(r0 + (mv ? ra : 0)) * rstride;
      const uint16_t *hp = reinterpret_cast<const uint16_t *>(arow);
      const uint16_t *lp = hp + F;
#pragma unroll
      for (int jj = 0; jj < NQ; ++jj) xpose4(w[j].w[jj]);
      // one partial per block-quad, each summed from zero over its four
      // blocks, the same partials the down kernel's waves form
#pragma unroll
      for (int jj = 0; jj < NQ; ++jj) {
        f32x4_t acc = zero4;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int b = ha * NBh + 4 * jj + p;  // block of this lane's A row
          const Vec ah = mv ? Fm::a_plane(hp, b, g) : Fm::zero();
          const Vec al = mv ? Fm::a_plane(lp, b, g) : Fm::zero();
          const Vec bw = Fm::b_w(word(w[j].w[jj], p));
          if constexpr (kInt4) {
            f32x4_t c0v = Fm::mfma(ah, cvec, zero4);
            c0v = Fm::mfma(al, cvec, c0v);
            f32x4_t c = Fm::mfma(ah, bw, c0v);
            c = Fm::mfma(al, bw, c);
            acc = fma4(scale4(w[j].s[jj][0], w[j].s[jj][1], p), c, acc);
          } else {
            acc = Fm::mfma(ah, bw, acc);
            acc = Fm::mfma(al, bw, acc);
          }
        }
        if constexpr (!kInt4) acc = acc * w[j].rs;
        // lane (n, g) holds tile rows 4g..4g+3 of column n: kept where the
        // row's half (g >> 1) is the column's half
        if ((g >> 1) == hb) {
          const int q = hb * NQ + jj;  // quad of the row
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 4 * (g & 1) + i;
            if (r < nr) pout[(q * n_rows_all + r0 + r) * kDcFeat + (n & 7)] = acc[i];
          }
        }
      }
    }
  };

  // --- First batch of requests: the unit table (for the weight addresses), the slots, the
  // rows' routing weights and every SwiGLU row of the call.  The weights
  // are requested as soon as the table has arrived, before the staged rows
  // are stored, so both travel together.
  __shared__ int slot_pos[8 * kDcMaxK];
  __shared__ float row_wt[8 * kDcMaxK];
  const int TK = T * K;
  const bool slot_thread = tid < TK;  // TK <= n_rows: also a row thread
  int my_pos = 0;
  float my_rw = 0.f;
  if (slot_thread) {
    my_pos = d.inv_pos[tid];
    my_rw = a.row_w[tid];
  }
  const int pieces_row = F / 4;  // 16-byte pieces per row (hi + lo planes)
  const int total = n_rows_all * pieces_row;
  const uint4 *src = reinterpret_cast<const uint4 *>(a.act);
  // named values rather than an array, which would live in scratch; a piece
  // past the end re-reads (and later rewrites) the last one
#define DC_PIECE(b) \
  const int i##b = min(tid + (b) * nthr, total - 1); \
  const uint4 v##b = src[i##b];
  DC_PIECE(0) DC_PIECE(1) DC_PIECE(2) DC_PIECE(3) DC_PIECE(4) DC_PIECE(5) DC_PIECE(6) DC_PIECE(7)
#undef DC_PIECE
  issue(0);
  auto put = [&](int i, const uint4 &v) {
    const int r = i / pieces_row, c = i - r * pieces_row;
    *reinterpret_cast<uint4 *>(act_l + static_cast<size_t>(r) * rstride + 16 * c) = v;
  };
  put(i0, v0);
  put(i1, v1);
  put(i2, v2);
  put(i3, v3);
  put(i4, v4);
  put(i5, v5);
  put(i6, v6);
  put(i7, v7);
  if (slot_thread) {
    slot_pos[tid] = my_pos;
    row_wt[tid] = my_rw;
  }
  lds_barrier();
  compute(0);
  for (int c0 = W * kDcUpw; c0 < n_units; c0 += W * kDcUpw) {
    issue(c0);
    compute(c0);
  }
  lds_barrier();

  // --- Combine, as the two-launch path does it.  First every row (p, f):
  // its quads' partials added in quad order, a routed row then multiplied by
  // its routing weight (rounded as when it is stored); left in place of its
  // first partial.
  for (int i = tid; i < n_rows_all * kDcFeat; i += nthr) {
    const int p = i / kDcFeat, f = i - p * kDcFeat;
    float v = pout[i];
#pragma unroll
    for (int q = 1; q < 2 * NQ; ++q) v += pout[(q * n_rows_all + p) * kDcFeat + f];
    if (p < a.n_rows) v *= row_wt[p];
    pout[i] = v;
  }
  lds_barrier();
  // then thread (t, f) < (T, 8): token t's slot rows in slot order, then the
  // shared expert's row
  if (tid < T * kDcFeat) {
    const int ct = tid / kDcFeat, cf = tid - ct * kDcFeat;
    // every read unconditional (clamped), then the selection
    int pos[kDcMaxK];
    float vals[kDcMaxK];
#pragma unroll
    for (int k = 0; k < kDcMaxK; ++k) pos[k] = slot_pos[ct * K + min(k, K - 1)];
#pragma unroll
    for (int k = 0; k < kDcMaxK; ++k) vals[k] = pout[min(max(pos[k], 0), a.n_rows - 1) * kDcFeat + cf];
    float y = 0.f;
#pragma unroll
    for (int k = 0; k < kDcMaxK; ++k)
      if (k < K && pos[k] >= 0 && pos[k] < a.n_rows) y += vals[k];
    if (has_shared) {
      // the shared row, scaled by its gate when there is one, exactly as
      // the combine kernel adds it
      const float sv = pout[(a.n_rows + ct) * kDcFeat + cf];
      y = d.shared_gate ? fmaf(d.shared_gate[ct], sv, y) : y + sv;
    }
    const size_t o = static_cast<size_t>(ct) * H + h0 + cf;
    d.y[o] = y;
    if (d.residual_out) d.residual_out[o] = f32_to_bf16_rne(bf16_to_f32(d.residual_in[o]) + y);
  }
}

// Waves of a block: one per unit when the units fit (the shared expert and
// at most max_units routed ones), else 16 that loop over the units.
static int dc_waves(const FfnArgs &a) {
  const int units = a.max_units + (a.Fs > 0 ? 1 : 0);
  return units < kDcMaxThreads / 64 ? units : kDcMaxThreads / 64;
}

size_t down_combine_lds(const FfnArgs &a) {
  const size_t rows = static_cast<size_t>(a.n_rows) + (a.Fs > 0 ? a.T : 0);
  const int nq = a.F / (a.fmt == MOE_W_INT4_B32 ? 32 : 16) / 8;
  return rows * dc_row_bytes(a.F) + 2 * nq * rows * kDcFeat * sizeof(float);
}

bool down_combine_ok(const FfnArgs &a, int K) {
  const int bk = a.fmt == MOE_W_INT4_B32 ? 32 : 16;
  if (a.fmt != MOE_W_INT4_B32 && a.fmt != MOE_W_INT8_ROW) return false;
  if (a.F % (8 * bk)) return false;
  const int nq = a.F / bk / 8;  // block-quads per half row
  return a.T >= 1 && a.T <= 8 && (nq == 2 || nq == 4) && a.H % kDcFeat == 0 &&
         (a.Fs == 0 || a.Fs == a.F) && K >= 1 && K <= kDcMaxK && a.max_units >= 1 &&
         down_combine_lds(a) <= kDcLdsBytes &&
         (a.n_rows + (a.Fs > 0 ? a.T : 0)) * (a.F / 4) <= kDcStage * 64 * dc_waves(a);
}

template <int FMT, int NQ>
static hipError_t launch_dc_t(const DownCombineArgs &d, hipStream_t s) {
  const size_t lds = down_combine_lds(d.f);
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&down_combine_kernel<FMT, NQ>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  return launch_kernel(down_combine_kernel<FMT, NQ>, dim3(d.f.H / kDcFeat), dim3(64 * dc_waves(d.f)),
                       static_cast<uint32_t>(lds), s, d.f.ev, d);
}

template <int FMT>
static hipError_t launch_dc_f(const DownCombineArgs &d, hipStream_t s) {
  const int nq = d.f.F / (FMT == MOE_W_INT4_B32 ? 32 : 16) / 8;
  if (nq == 2) return launch_dc_t<FMT, 2>(d, s);
  return launch_dc_t<FMT, 4>(d, s);
}

hipError_t launch_down_combine(const DownCombineArgs &d, hipStream_t s) {
  if (!down_combine_ok(d.f, d.K)) return hipErrorInvalidValue;
  return d.f.fmt == MOE_W_INT4_B32 ? launch_dc_f<MOE_W_INT4_B32>(d, s) : launch_dc_f<MOE_W_INT8_ROW>(d, s);
}

}  // namespace moe
