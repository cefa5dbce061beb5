// Router: logits = x Wr^T (+ bias) in float32, then a wavefront top-k with
// the lowest-index tie rule and the routing weights.
//
// The pages fold "router top-k and grouping" into one launch on their card
// ("Qwen3.6-35B-A3B: pictures, several requests at once and speed", Speed
// (0.1.45)) after a one-thread walk over the 256 experts proved slow; here a
// whole wavefront holds a token's E logits (E/64 per lane, each lane's
// sorted once) and each of the K rounds is one wave-wide maximum of the
// lanes' leading logits, done with DPP row steps and four lane reads.  Equal
// logits go to the lower expert index, the rule the pages apply to their own
// arg-max ("Models and backends", What was tuned).
#include <float.h>
#include <math.h>

#include "mfma_common.h"
#include "route_common.h"

namespace moe {

constexpr int kRouterTokens = 16;  // tokens per block (x tile staged in LDS)

// Router arithmetic shared by every router kernel, so that all of them give
// the same bits: H is cut into slices of Hs elements; a slice's partial
// logit for (token t, expert e) is computed by the wave owning e, lane
// (t, g) summing elements 16 i + 4 g + {0..3} of the slice in order, the
// four lanes of a token then added as (g0 + g2) + (g1 + g3); the logit is
// ((0 + p_0) + p_1) + ... + p_{S-1}, plus the bias.

// Sum over the four rows of 16 lanes, in the order (r0 + r2) + (r1 + r3);
// every lane receives its column's sum.
MOE_DEV float rows4_sum(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const float a = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  const uint32_t ua = __float_as_uint(a);
  const auto q = __builtin_amdgcn_permlane16_swap(ua, ua, false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

// Stages the router rows of the block's 4 experts (slice [h0, h0 + Hs)) and
// the slice of nt token rows starting at token t0 into LDS.
// Row E is the shared expert's gate row when gate_w is given (the router
// and the shared gate as one product); rows past the last read row 0.
MOE_DEV void stage_router_slice(const float *__restrict__ router_w, const float *__restrict__ gate_w,
                                const uint16_t *__restrict__ x, int E, int H, int Hs, int e0, int h0, int t0, int nt,
                                float *wr_l, uint16_t *xs) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int e = e0 + wave;
  const float *row = e < E ? router_w + static_cast<size_t>(e) * H : (gate_w && e == E ? gate_w : router_w);
  const float4 *src = reinterpret_cast<const float4 *>(row + h0);
  float4 *dst = reinterpret_cast<float4 *>(wr_l + wave * Hs);
  const int n4 = Hs / 256;  // float4 per lane, <= kFusedMaxChunks
  float4 v[kFusedMaxChunks];
#pragma unroll
  for (int c = 0; c < kFusedMaxChunks; ++c) v[c] = c < n4 ? src[c * 64 + lane] : make_float4(0.f, 0.f, 0.f, 0.f);
  const int per_row = Hs / 8;
  const int n8 = nt * per_row;  // <= 256 * kStageBatch
  const int xstride = Hs + 8;
  uint4 xv[kStageBatch];
#pragma unroll
  for (int b = 0; b < kStageBatch; ++b) {
    const int i = tid + 256 * b;
    const int t = i / per_row, k = i - t * per_row;
    // unconditional assignment keeps the batch in registers
    xv[b] = i < n8 ? reinterpret_cast<const uint4 *>(x + static_cast<size_t>(t0 + t) * H + h0)[k]
                   : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int c = 0; c < kFusedMaxChunks; ++c)
    if (c < n4) dst[c * 64 + lane] = v[c];
#pragma unroll
  for (int b = 0; b < kStageBatch; ++b) {
    const int i = tid + 256 * b;
    if (i < n8) {
      const int t = i / per_row, k = i - t * per_row;
      reinterpret_cast<uint4 *>(xs + t * xstride)[k] = xv[b];
    }
  }
}

// Partial logit of one staged slice for the calling wave's expert; lane
// (t = lane & 15, g = lane >> 4); every lane of column t gets token t's sum.
MOE_DEV float slice_partial(const float *wrow, const uint16_t *xs, int Hs, int nt, bool valid) {
  const int lane = __lane_id();
  const int t = lane & 15, g = lane >> 4;
  float acc = 0.f;
  if (valid && t < nt) {
    const uint16_t *xrow = xs + t * (Hs + 8);
    for (int i = 0; i < Hs / 16; ++i) {
      const float4 w4 = *reinterpret_cast<const float4 *>(wrow + 16 * i + 4 * g);
      const uint2 x4 = *reinterpret_cast<const uint2 *>(xrow + 16 * i + 4 * g);
      acc = fmaf(w4.x, bf16_lo(x4.x), acc);
      acc = fmaf(w4.y, bf16_hi(x4.x), acc);
      acc = fmaf(w4.z, bf16_lo(x4.y), acc);
      acc = fmaf(w4.w, bf16_hi(x4.y), acc);
    }
  }
  return rows4_sum(acc);
}

size_t router_slice_lds_bytes(int Hs, int tokens) {
  return static_cast<size_t>(4) * Hs * 4 + static_cast<size_t>(tokens) * (Hs + 8) * 2;
}

// One block per (4 experts, 16 tokens); the slices are visited in order.
// With gate_w, expert row E is the shared gate row: gate[t] receives the
// sigmoid of its logit (no bias).
__global__ void __launch_bounds__(256) router_logits_kernel(const float *__restrict__ wr,
                                                            const float *__restrict__ bias,
                                                            const uint16_t *__restrict__ x, int32_t T, int32_t H,
                                                            int32_t E, float *__restrict__ logits,
                                                            const float *__restrict__ gate_w,
                                                            float *__restrict__ gate) {
  extern __shared__ float4 smem_router[];
  const int Hs = route_fused_slice(H);
  float *wr_l = reinterpret_cast<float *>(smem_router);
  uint16_t *xs = reinterpret_cast<uint16_t *>(wr_l + 4 * Hs);
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int e0 = blockIdx.x * 4;
  const int e = e0 + wave;
  const int t0 = blockIdx.y * kRouterTokens;
  const int nt = min(kRouterTokens, T - t0);
  float total = 0.f;
  for (int h0 = 0; h0 < H; h0 += Hs) {
    lds_barrier();  // the previous slice's readers are done
    stage_router_slice(wr, gate_w, x, E, H, Hs, e0, h0, t0, nt, wr_l, xs);
    lds_barrier();
    total += slice_partial(wr_l + wave * Hs, xs, Hs, nt, e < E || (gate_w && e == E));
  }
  if (e < E && lane < nt) logits[static_cast<size_t>(t0 + lane) * E + e] = total + (bias ? bias[e] : 0.f);
  if (gate_w && e == E && lane < nt) gate[t0 + lane] = 1.f / (1.f + expf(-total));
}

// ---------------------------------------------------------- large batches
//
// For more than kFusedTokens tokens the logits are a GEMM on the bf16 matrix
// cores with fp32 accuracy: x is exact in bf16, and each fp32 router weight
// w is split exactly into three bf16 parts, w = hi + mid + lo (hi: w cut to
// 8 significant bits, mid: the remainder cut likewise, lo: the last 8 bits),
// so three v_mfma_f32_32x32x16_bf16 per 16-wide k-step form every product
// exactly and accumulate it in fp32, as an fp32 dot product does (in another
// order).  The reduction is split into kRgSlices slices: a block owns 64
// tokens x 64 experts over one slice and writes its partial sums; the
// top-k kernel adds the slices in order (then the bias), so a weight row is
// read by T / 64 blocks and the x rows by E / 64.  Both operands go from
// global memory straight into LDS by direct loads, one 64-wide k-step ahead
// in two buffers; the block then splits the step's weights once into three
// bf16 planes in LDS (no wave splits a weight another wave splits too).
// Each of the 4 waves owns one 32x32 tile (tokens 32 (w & 1), experts
// 32 (w >> 1)); the 72 KB of LDS let two blocks share a compute unit, so one
// block's loads overlap the other's matrix work.  moe_route and the layer
// use this kernel alike for such batches.
constexpr int kRgTok = 64, kRgExp = 64, kRgStep = 64, kRgSlices = 4;
constexpr int kRgThreads = 256;

typedef __bf16 rbf16x8_t __attribute__((ext_vector_type(8)));
typedef float rf32x16_t __attribute__((ext_vector_type(16)));

// eight fp32 weights -> their hi, mid and lo bf16 parts, pairs in k order
MOE_DEV void split3(const float4 &w0, const float4 &w1, u32x4_t &hi, u32x4_t &mid, u32x4_t &lo) {
  const float w[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
  uint32_t ph[8], pm[8], pl[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t h = __float_as_uint(w[i]) & 0xFFFF0000u;
    const float r1 = w[i] - __uint_as_float(h);  // exact
    const uint32_t m = __float_as_uint(r1) & 0xFFFF0000u;
    const float r2 = r1 - __uint_as_float(m);  // exact, at most 8 significant bits
    ph[i] = h;
    pm[i] = m;
    pl[i] = __float_as_uint(r2);  // its low 16 bits are zero
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // (element 2i in the low half, 2i + 1 in the high half)
    hi[i] = __builtin_amdgcn_perm(ph[2 * i + 1], ph[2 * i], 0x07060302u);
    mid[i] = __builtin_amdgcn_perm(pm[2 * i + 1], pm[2 * i], 0x07060302u);
    lo[i] = __builtin_amdgcn_perm(pl[2 * i + 1], pl[2 * i], 0x07060302u);
  }
}

MOE_DEV rf32x16_t mfma32_bf16(const u32x4_t &a, const u32x4_t &b, const rf32x16_t &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(rbf16x8_t, a), __builtin_bit_cast(rbf16x8_t, b),
                                                 c, 0, 0, 0);
}

// part[slice][t][e] = sum of x[t][k] w[e][k] over the slice's k (no bias);
// the blocks of expert block 0 also write x in fp16, pair-permuted (the
// prefill expert GEMMs' operand form).  SPS = steps of kRgStep per slice.
template <int SPS>
__global__ void __launch_bounds__(kRgThreads) router_gemm_kernel(const float *__restrict__ wr,
                                                                 const uint16_t *__restrict__ x, int32_t T,
                                                                 int32_t H, int32_t E, float *__restrict__ part,
                                                                 uint16_t *__restrict__ x16) {
  // raw step operands, two buffers: x rows [64][8 pieces of 8 bf16] and
  // weight rows [64][16 pieces of 4 fp32]; the split weights [3][64][8]
  __shared__ uint4 rg_x0[kRgTok * 8], rg_x1[kRgTok * 8];
  __shared__ uint4 rg_w0[kRgExp * 16], rg_w1[kRgExp * 16];
  __shared__ uint4 rg_p[3][kRgExp * 8];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int c = lane & 31, g = lane >> 5;
  const int tt = wave & 1, eq = wave >> 1;  // this wave's token tile and expert tile
  const int t0 = blockIdx.x * kRgTok, e0 = blockIdx.y * kRgExp;
  const int slice = blockIdx.z;
  const int k0 = slice * SPS * kRgStep;
  auto xbuf = [&](int b) __attribute__((always_inline)) { return b == 0 ? rg_x0 : rg_x1; };
  auto wbuf = [&](int b) __attribute__((always_inline)) { return b == 0 ? rg_w0 : rg_w1; };
  // direct loads: instruction i of wave w fills x rows 8 (4 i + w) + l / 8,
  // slot l % 8 holding piece slot ^ (row & 7), and weight rows
  // 4 (4 w + i) + l / 16, slot l % 16 holding piece slot ^ (row & 15).  Rows
  // past T or E read row 0: their sums land in outputs never stored.
  gchar_t *xg = uniform_gptr(x);
  gchar_t *wg = uniform_gptr(wr);
  uint32_t xoff[2], woff[4];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 8 * (4 * i + wave) + (lane >> 3);
    xoff[i] = (static_cast<uint32_t>(t0 + r < T ? t0 + r : 0) * H + k0) * 2 + 16 * ((lane & 7) ^ (r & 7));
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * (4 * wave + i) + (lane >> 4);
    woff[i] = (static_cast<uint32_t>(e0 + r < E ? e0 + r : 0) * H + k0) * 4 + 16 * ((lane & 15) ^ (r & 15));
  }
  auto load_step = [&](int s) __attribute__((always_inline)) {
    const int b = s & 1;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      __builtin_amdgcn_global_load_lds(xg + (xoff[i] + static_cast<uint32_t>(2 * kRgStep) * s),
                                       (__attribute__((address_space(3))) void *)(xbuf(b) + 64 * (4 * i + wave)), 16,
                                       0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_global_load_lds(wg + (woff[i] + static_cast<uint32_t>(4 * kRgStep) * s),
                                       (__attribute__((address_space(3))) void *)(wbuf(b) + 64 * (4 * wave + i)), 16,
                                       0, 0);
  };
  // the block's split of a step's weights: thread (row tid / 4, quarter
  // tid % 4) splits k 16 q .. 16 q + 15 of its row into the planes' pieces
  // 2 q and 2 q + 1 (slot piece ^ (row & 7))
  auto split_step = [&](int b) __attribute__((always_inline)) {
    const int r = tid >> 2, q = tid & 3;
    const uint4 *src = wbuf(b) + 16 * r;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int pc = 4 * q + 2 * hh;  // fp32 pieces pc, pc + 1: k 8 (2 q + hh) .. + 7
      const uint4 a0 = src[pc ^ (r & 15)], a1 = src[(pc + 1) ^ (r & 15)];
      u32x4_t ph, pm, pl;
      split3(make_float4(__uint_as_float(a0.x), __uint_as_float(a0.y), __uint_as_float(a0.z), __uint_as_float(a0.w)),
             make_float4(__uint_as_float(a1.x), __uint_as_float(a1.y), __uint_as_float(a1.z), __uint_as_float(a1.w)),
             ph, pm, pl);
      const int slot = (2 * q + hh) ^ (r & 7);
      rg_p[0][8 * r + slot] = make_uint4(ph[0], ph[1], ph[2], ph[3]);
      rg_p[1][8 * r + slot] = make_uint4(pm[0], pm[1], pm[2], pm[3]);
      rg_p[2][8 * r + slot] = make_uint4(pl[0], pl[1], pl[2], pl[3]);
    }
  };
  // the fp16 copy of x: thread (row 8 (4 i + w) + l / 8, slot l % 8) writes
  // the piece it loaded (blocks of expert block 0 only)
  const bool write16 = x16 && blockIdx.y == 0;
  rf32x16_t acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
  const int ar = 32 * tt + c, er = 32 * eq + c;  // this lane's x row and weight row
  load_step(0);
  __builtin_amdgcn_sched_barrier(0);
  if (SPS > 1) load_step(1);
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(SPS > 1 ? 6 : 0));
  lds_barrier();
  split_step(0);
  lds_barrier();
  auto step = [&](auto sc) __attribute__((always_inline)) {
    constexpr int s = decltype(sc)::value;
    constexpr int b = s & 1;
    if (write16) {
      // this thread's landed x pieces, in fp16 operand order
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = 8 * (4 * i + wave) + (lane >> 3);
        if (t0 + r < T) {
          const int pcs = (lane & 7) ^ (r & 7);
          const uint4 v = xbuf(b)[64 * (4 * i + wave) + lane];
          const u32x4_t pp = pair_permute(v);
          *reinterpret_cast<uint4 *>(x16 + static_cast<size_t>(t0 + r) * H + k0 + kRgStep * s + 8 * pcs) =
              make_uint4(bf16x2_to_f16x2(pp.x), bf16x2_to_f16x2(pp.y), bf16x2_to_f16x2(pp.z),
                         bf16x2_to_f16x2(pp.w));
        }
      }
    }
#pragma unroll
    for (int kk = 0; kk < kRgStep / 16; ++kk) {
      const int pc = 2 * kk + g;  // the lane's 8 k of the 16-wide step
      const uint4 av = xbuf(b)[8 * ar + (pc ^ (ar & 7))];
      const u32x4_t A = {av.x, av.y, av.z, av.w};
#pragma unroll
      for (int pl = 0; pl < 3; ++pl) {
        const uint4 bv = rg_p[pl][8 * er + (pc ^ (er & 7))];
        const u32x4_t B = {bv.x, bv.y, bv.z, bv.w};
        acc = mfma32_bf16(A, B, acc);
      }
    }
    if constexpr (s + 1 < SPS) {
      lds_barrier();  // every wave is done with the planes and with buffer b
      if constexpr (s + 2 < SPS) load_step(s + 2);
      __builtin_amdgcn_sched_barrier(0);
      // step s + 1 has landed once at most step s + 2's six requests are pending
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(s + 2 < SPS ? 6 : 0));
      lds_barrier();
      split_step(b ^ 1);
      lds_barrier();
    }
  };
  unrolled_steps(std::make_integer_sequence<int, SPS>{}, step);
  // result (m, n) of the 32x32 tile sits in lane n + 32 ((m / 4) % 2),
  // register 4 (m / 8) + m % 4
  const int e = e0 + er;
  if (e < E) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int t = t0 + 32 * tt + 8 * (j >> 2) + 4 * g + (j & 3);
      if (t < T) part[(static_cast<size_t>(slice) * T + t) * E + e] = acc[j];
    }
  }
}

// One wave per token.  Lane l holds experts l, l+64, ... (up to 16 each).
// With gate_w (a call whose logits came from the matrix-core GEMM) the wave
// also forms its token's shared gate logit, lane l summing elements
// l, l + 64, ... and the wave adding the lanes in a fixed order, and writes
// its sigmoid to gate[t].
//
// The logits come either whole (S = 1, bias already added) or as S partial
// sums [S][T][E] from the router GEMM, added here in slice order and then
// the bias; logits_out (or NULL) then receives them.
template <int NPL>
__global__ void __launch_bounds__(256) topk_kernel(const float *__restrict__ logits, int32_t S,
                                                   const float *__restrict__ bias, float *__restrict__ logits_out,
                                                   int32_t T, int32_t E, int32_t K, int32_t renorm,
                                                   int32_t *__restrict__ ids, float *__restrict__ wout,
                                                   const uint16_t *__restrict__ x, int32_t H,
                                                   const float *__restrict__ gate_w, float *__restrict__ gate) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  if (gate_w) {
    const uint16_t *xr = x + static_cast<size_t>(t) * H;
    float acc = 0.f;
    for (int h = lane; h < H; h += 64) acc = fmaf(gate_w[h], bf16_to_f32(xr[h]), acc);
    const float z = sum64(acc);
    if (lane == 0) gate[t] = 1.f / (1.f + expf(-z));
  }
  float v[NPL];
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    const int e = lane + 64 * j;
    float val = -INFINITY;
    if (e < E) {
      // every slice requested at once, then added in order
      float pv[kRgSlices];
#pragma unroll
      for (int sl = 0; sl < kRgSlices; ++sl)
        pv[sl] = sl < S ? logits[(static_cast<size_t>(sl) * T + t) * E + e] : 0.f;
      float sum = pv[0];
#pragma unroll
      for (int sl = 1; sl < kRgSlices; ++sl)
        if (sl < S) sum += pv[sl];
      if (S > 1) {
        if (bias) sum += bias[e];
        if (logits_out) logits_out[static_cast<size_t>(t) * E + e] = sum;
      }
      val = sum == sum ? sum : -INFINITY;  // NaN never outranks a number
    }
    v[j] = val;
  }
  int my_e;
  float my_w;
  wave_topk<NPL>(v, E, K, renorm, my_e, my_w);
  if (lane < K) {
    ids[static_cast<size_t>(t) * K + lane] = my_e;
    wout[static_cast<size_t>(t) * K + lane] = my_w;
  }
}

// ------------------------------------------------------- decode routing
//
// For a decode batch (T <= kFusedTokens) routing takes two launches: the
// pages merge "router top-k and grouping" into one kernel ("Qwen3.6-35B-A3B:
// pictures, several requests at once and speed", Speed (0.1.45)); here the
// router's blocks (4 experts x one slice of H each) write partial logits,
// and one block then adds the slices in a fixed order, selects the top-k of
// every token and builds the permutation.  (A last-block hand-off inside
// one launch would need a device-scope fence per block, which on this chip
// writes back the issuing XCD's L2 and costs far more than a launch.)

__global__ void __launch_bounds__(256) route_partial_kernel(RouteFusedArgs a) {
  extern __shared__ float4 smem_route[];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int T = a.T, E = a.E, H = a.H, Hs = a.Hs, S = a.S, Ep = a.Ep;
  const int slice = blockIdx.x % S;
  const int e = (blockIdx.x / S) * 4 + wave;  // e == E: the shared gate row (Ep = E + 1)
  const int h0 = slice * Hs;
  float *wr_l = reinterpret_cast<float *>(smem_route);        // [4][Hs]
  uint16_t *xs = reinterpret_cast<uint16_t *>(wr_l + 4 * Hs);  // [T][Hs + 8]
  stage_router_slice(a.router_w, a.gate_w, a.x, E, H, Hs, e - wave, h0, 0, T, wr_l, xs);
  lds_barrier();
  const float p = slice_partial(wr_l + wave * Hs, xs, Hs, T, e < Ep);
  if (lane < T && e < Ep) a.part[(static_cast<size_t>(slice) * T + lane) * Ep + e] = p;
}

// One block of kSelectThreads: the routing of a decode batch (top-k and
// permutation) from the partial logits, published to global memory.
constexpr int kSelectThreads = 1024;

template <int NPL>
__global__ void __launch_bounds__(kSelectThreads) route_select_kernel(RouteFusedArgs a) {
  __shared__ RouteLds L;
  if constexpr (NPL <= 4)
    route_in_block_small<NPL>(a, L, true);
  else
    route_in_block<NPL>(a, L, true);
}

hipError_t launch_route_partial(const RouteFusedArgs &a, hipStream_t s) {
  const int groups = (a.Ep + 3) / 4;
  route_partial_kernel<<<groups * a.S, 256, router_slice_lds_bytes(a.Hs, a.T), s>>>(a);
  return hipGetLastError();
}

hipError_t launch_route_fused(const RouteFusedArgs &a, hipStream_t s) {
  hipError_t err = launch_route_partial(a, s);
  if (err != hipSuccess) return err;
  const int npl = (a.E + 63) / 64;
  if (npl <= 1)
    route_select_kernel<1><<<1, kSelectThreads, 0, s>>>(a);
  else if (npl <= 2)
    route_select_kernel<2><<<1, kSelectThreads, 0, s>>>(a);
  else if (npl <= 4)
    route_select_kernel<4><<<1, kSelectThreads, 0, s>>>(a);
  else
    route_select_kernel<16><<<1, kSelectThreads, 0, s>>>(a);
  return hipGetLastError();
}

// Steps of the router GEMM per slice (H = kRgSlices * steps * kRgStep),
// or 0 where the call takes the partial-logit router kernel.
static int router_gemm_steps(int T, int H, int path) {
  const bool many = path == kPathPrefill || (path == kPathAuto && T > kFusedTokens);
  if (!many || H % (kRgSlices * kRgStep)) return 0;
  const int sps = H / (kRgSlices * kRgStep);
  return (sps == 2 || sps == 4 || sps == 8 || sps == 16) ? sps : 0;
}

static bool router_mfma_ok(const RouteArgs &a) { return router_gemm_steps(a.T, a.H, a.path) > 0; }

size_t router_partial_floats(int T, int H, int E, int path) {
  return router_gemm_steps(T, H, path) > 0 ? static_cast<size_t>(kRgSlices) * T * E : 0;
}

bool router_writes_x16(const RouteArgs &a) { return a.x16 != nullptr && router_mfma_ok(a); }

hipError_t launch_router_logits(const RouteArgs &a, hipStream_t s) {
  const int sps = router_gemm_steps(a.T, a.H, a.path);
  if (sps > 0) {
    if (!a.part) return hipErrorInvalidValue;
    dim3 g((a.T + kRgTok - 1) / kRgTok, (a.E + kRgExp - 1) / kRgExp, kRgSlices);
#define MOE_RG(N) router_gemm_kernel<N><<<g, kRgThreads, 0, s>>>(a.router_w, a.x, a.T, a.H, a.E, a.part, a.x16)
    if (sps == 2)
      MOE_RG(2);
    else if (sps == 4)
      MOE_RG(4);
    else if (sps == 8)
      MOE_RG(8);
    else
      MOE_RG(16);
#undef MOE_RG
    return hipGetLastError();
  }
  const int rows = a.E + (a.gate_w ? 1 : 0);  // the gate row rides with the router rows
  dim3 grid((rows + 3) / 4, (a.T + kRouterTokens - 1) / kRouterTokens);
  const size_t lds = router_slice_lds_bytes(route_fused_slice(a.H), kRouterTokens);
  router_logits_kernel<<<grid, 256, lds, s>>>(a.router_w, a.router_bias, a.x, a.T, a.H, a.E, a.logits, a.gate_w,
                                              a.gate);
  return hipGetLastError();
}

hipError_t launch_topk(const RouteArgs &a, hipStream_t s) {
  dim3 grid((a.T + 3) / 4);
  const int npl = (a.E + 63) / 64;
  // the shared gate is formed here only when the router GEMM left it out
  const bool gemm = router_mfma_ok(a);
  const float *gw = gemm ? a.gate_w : nullptr;
  const float *in = gemm ? a.part : a.logits;
  const int S = gemm ? kRgSlices : 1;
#define MOE_TOPK(N)                                                                                                  \
  topk_kernel<N><<<grid, 256, 0, s>>>(in, S, a.router_bias, a.logits, a.T, a.E, a.K, a.renorm, a.ids, a.w, a.x, a.H, \
                                      gw, a.gate)
  if (npl <= 1)
    MOE_TOPK(1);
  else if (npl <= 2)
    MOE_TOPK(2);
  else if (npl <= 4)
    MOE_TOPK(4);
  else if (npl <= 8)
    MOE_TOPK(8);
  else
    MOE_TOPK(16);
#undef MOE_TOPK
  return hipGetLastError();
}

}  // namespace moe
