// Router: logits = x Wr^T (+ bias) in float32, then a wavefront top-k with
// the lowest-index tie rule and the routing weights.
//
// The pages fold "router top-k and grouping" into one launch on their card
// ("Qwen3.6-35B-A3B: pictures, several requests at once and speed", Speed
// (0.1.45)) after a one-thread walk over the 256 experts proved slow; here a
// whole wavefront holds a token's E logits (E/64 per lane) and each of the K
// rounds is one wave-wide arg-max done with DPP row steps and four lane
// reads.  Equal logits go to the lower expert index, the rule the pages
// apply to their own arg-max ("Models and backends", What was tuned): the
// arg-max runs on 64-bit keys (order-preserving float bits, inverted index).
#include <float.h>
#include <math.h>

#include "common.h"

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
MOE_DEV void stage_router_slice(const float *__restrict__ router_w, const uint16_t *__restrict__ x, int E, int H,
                                int Hs, int e0, int h0, int t0, int nt, float *wr_l, uint16_t *xs) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int e = e0 + wave;
  const float4 *src = reinterpret_cast<const float4 *>(router_w + static_cast<size_t>(e < E ? e : 0) * H + h0);
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
__global__ void __launch_bounds__(256) router_logits_kernel(const float *__restrict__ wr,
                                                            const float *__restrict__ bias,
                                                            const uint16_t *__restrict__ x, int32_t T, int32_t H,
                                                            int32_t E, float *__restrict__ logits) {
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
    stage_router_slice(wr, x, E, H, Hs, e0, h0, t0, nt, wr_l, xs);
    lds_barrier();
    total += slice_partial(wr_l + wave * Hs, xs, Hs, nt, e < E);
  }
  if (e < E && lane < nt) logits[static_cast<size_t>(t0 + lane) * E + e] = total + (bias ? bias[e] : 0.f);
}

// Order-preserving map of a float onto uint32 (NaN must be excluded).
MOE_DEV uint32_t float_key(float v) {
  const uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
MOE_DEV float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

template <int CTRL>
MOE_DEV uint32_t dpp_u32(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xF, 0xF, true));
}

// Wave-wide maximum (uniform result).
MOE_DEV uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<0xB1>(v));   // quad_perm [1,0,3,2]
  v = max(v, dpp_u32<0x4E>(v));   // quad_perm [2,3,0,1]
  v = max(v, dpp_u32<0x141>(v));  // row_half_mirror
  v = max(v, dpp_u32<0x140>(v));  // row_mirror
  const uint32_t a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
  const uint32_t c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
  return max(max(a, b), max(c, d));
}

// Top-k of one token's logits held by a whole wave: lane l holds experts
// l, l+64, ... in v[] (NaN already replaced by -inf, absent experts -inf).
// Lane k < K receives round k's expert and routing weight.
template <int NPL>
MOE_DEV void wave_topk(const float (&v)[NPL], int32_t E, int32_t K, int32_t renorm, int &my_e, float &my_w) {
  const int lane = __lane_id();
  uint32_t key[NPL];  // 0 = used or absent
#pragma unroll
  for (int j = 0; j < NPL; ++j) key[j] = (lane + 64 * j < E) ? float_key(v[j]) : 0u;
  float top_v = 0.f;
  float my_v = 0.f;  // lane k keeps round k's value and index
  my_e = 0;
  for (int k = 0; k < K; ++k) {
    // the largest remaining key, then the lowest expert index holding it
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < NPL; ++j) m = max(m, key[j]);
    m = wave_max_u32(m);
    int sel = 0;
#pragma unroll
    for (int j = NPL - 1; j >= 0; --j) {
      const uint64_t hit = __ballot(key[j] == m);
      if (hit) sel = 64 * j + __builtin_ctzll(hit);
    }
    if ((sel & 63) == lane) {
#pragma unroll
      for (int j = 0; j < NPL; ++j)
        if (j == (sel >> 6)) key[j] = 0u;
    }
    const float sel_v = key_float(m);
    if (k == 0) top_v = sel_v;
    if (lane == k) {
      my_v = sel_v;
      my_e = sel;
    }
  }
  // Softmax over the selected logits (renorm) or over all E, the largest
  // logit subtracted for range; sums in a fixed order.
  const float mine = (lane < K) ? expf(my_v - top_v) : 0.f;
  float denom;
  if (renorm) {
    denom = 0.f;
    for (int k = 0; k < K; ++k) denom += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mine), k));
  } else {
    float part = 0.f;
#pragma unroll
    for (int j = 0; j < NPL; ++j)
      if (lane + 64 * j < E) part += expf(v[j] - top_v);
    denom = sum64(part);
  }
  my_w = mine / denom;
}

// One wave per token.  Lane l holds experts l, l+64, ... (up to 16 each).
template <int NPL>
__global__ void __launch_bounds__(256) topk_kernel(const float *__restrict__ logits, int32_t T, int32_t E,
                                                   int32_t K, int32_t renorm, int32_t *__restrict__ ids,
                                                   float *__restrict__ wout) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  const float *l = logits + static_cast<size_t>(t) * E;
  float v[NPL];
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    const int e = lane + 64 * j;
    float val = -INFINITY;
    if (e < E) {
      val = l[e];
      if (val != val) val = -INFINITY;  // NaN never outranks a number
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
  const int T = a.T, E = a.E, H = a.H, Hs = a.Hs, S = a.S;
  const int slice = blockIdx.x % S;
  const int e = (blockIdx.x / S) * 4 + wave;
  const int h0 = slice * Hs;
  float *wr_l = reinterpret_cast<float *>(smem_route);        // [4][Hs]
  uint16_t *xs = reinterpret_cast<uint16_t *>(wr_l + 4 * Hs);  // [T][Hs + 8]
  stage_router_slice(a.router_w, a.x, E, H, Hs, e - wave, h0, 0, T, wr_l, xs);
  lds_barrier();
  const float p = slice_partial(wr_l + wave * Hs, xs, Hs, T, e < E);
  if (lane < T && e < E) a.part[(static_cast<size_t>(slice) * T + lane) * E + e] = p;
}

// Exclusive scan of one value per thread over the block (up to 16 waves);
// `scratch` holds 16 ints.  Also returns the block total.
MOE_DEV int block_scan(int v, int *scratch, int &total) {
  const int lane = __lane_id();
  const int wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  int inc = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(inc, off);
    if (lane >= off) inc += o;
  }
  if (lane == 63) scratch[wave] = inc;
  lds_barrier();
  int before = 0, all = 0;
  for (int w = 0; w < nw; ++w) {
    const int x = scratch[w];
    before += w < wave ? x : 0;
    all += x;
  }
  total = all;
  lds_barrier();
  return before + inc - v;
}

// One block of kSelectThreads: wave t adds token t's partial logits in
// order and selects its top-k; then the permutation of the T*K pairs
// (thread = expert for the counts and offsets, thread = pair for the rows).
constexpr int kSelectThreads = 1024;

template <int NPL>
__global__ void __launch_bounds__(kSelectThreads) route_select_kernel(RouteFusedArgs a) {
  extern __shared__ float4 smem_route[];
  __shared__ int scan_scratch[16];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int T = a.T, E = a.E, S = a.S, K = a.K;
  const int TK = T * K;
  int32_t *ids_l = reinterpret_cast<int32_t *>(smem_route);  // [TK]
  float *w_l = reinterpret_cast<float *>(ids_l + TK);         // [TK]
  int32_t *cnt = reinterpret_cast<int32_t *>(w_l + TK);       // [E]
  if (tid < E) cnt[tid] = 0;
  if (wave < T) {
    const int t = wave;
    // the partials of four slices at a time as independent loads, then
    // their sums in slice order
    const float *__restrict__ part = a.part;
    float acc[NPL];
#pragma unroll
    for (int j = 0; j < NPL; ++j) acc[j] = 0.f;
    for (int s0 = 0; s0 < S; s0 += 4) {
      float pv[NPL][4];
#pragma unroll
      for (int j = 0; j < NPL; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int ex = lane + 64 * j;
          pv[j][q] = (ex < E && s0 + q < S) ? part[(static_cast<size_t>(s0 + q) * T + t) * E + ex] : 0.f;
        }
#pragma unroll
      for (int j = 0; j < NPL; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (s0 + q < S) acc[j] += pv[j][q];
    }
    float v[NPL];
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const int ex = lane + 64 * j;
      const float sum = acc[j] + (a.router_bias && ex < E ? a.router_bias[ex] : 0.f);
      v[j] = (ex < E && sum == sum) ? sum : -INFINITY;  // NaN never outranks a number
      if (a.logits && ex < E) a.logits[static_cast<size_t>(t) * E + ex] = sum;
    }
    int my_e;
    float my_w;
    wave_topk<NPL>(v, E, K, a.renorm, my_e, my_w);
    if (lane < K) {
      const size_t p = static_cast<size_t>(t) * K + lane;
      a.ids[p] = my_e;
      a.w[p] = my_w;
      ids_l[p] = my_e;
      w_l[p] = my_w;
    }
  }
  lds_barrier();
  if (tid < TK) atomicAdd(&cnt[ids_l[tid]], 1);
  lds_barrier();
  const int c = tid < E ? cnt[tid] : 0;
  int total = 0, n_act = 0;
  const int base = block_scan(c, scan_scratch, total);
  const int abase = block_scan(c > 0 ? 1 : 0, scan_scratch, n_act);
  if (tid < E) {
    a.counts[tid] = c;
    a.offsets[tid] = base;
    if (c > 0) a.active[abase] = tid;
  }
  if (tid == 0) {
    a.offsets[E] = total;
    *a.n_active = n_act;
  }
  lds_barrier();          // every thread has read its count
  if (tid < E) cnt[tid] = base;  // cnt now holds the offsets
  lds_barrier();
  if (tid < TK) {
    const int ex = ids_l[tid];
    int r = 0;
    for (int q = 0; q < tid; ++q) r += ids_l[q] == ex;
    const int pos = cnt[ex] + r;
    a.row_tok[pos] = tid / K;
    a.row_w[pos] = w_l[tid];
    a.inv_pos[tid] = pos;
  }
}

hipError_t launch_route_fused(const RouteFusedArgs &a, hipStream_t s) {
  const int groups = (a.E + 3) / 4;
  route_partial_kernel<<<groups * a.S, 256, router_slice_lds_bytes(a.Hs, a.T), s>>>(a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const size_t lds = static_cast<size_t>(a.T) * a.K * 8 + static_cast<size_t>(a.E) * 4;
  const int npl = (a.E + 63) / 64;
  if (npl <= 1)
    route_select_kernel<1><<<1, kSelectThreads, lds, s>>>(a);
  else if (npl <= 2)
    route_select_kernel<2><<<1, kSelectThreads, lds, s>>>(a);
  else if (npl <= 4)
    route_select_kernel<4><<<1, kSelectThreads, lds, s>>>(a);
  else
    route_select_kernel<16><<<1, kSelectThreads, lds, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_router_logits(const RouteArgs &a, hipStream_t s) {
  dim3 grid((a.E + 3) / 4, (a.T + kRouterTokens - 1) / kRouterTokens);
  const size_t lds = router_slice_lds_bytes(route_fused_slice(a.H), kRouterTokens);
  router_logits_kernel<<<grid, 256, lds, s>>>(a.router_w, a.router_bias, a.x, a.T, a.H, a.E, a.logits);
  return hipGetLastError();
}

hipError_t launch_topk(const RouteArgs &a, hipStream_t s) {
  dim3 grid((a.T + 3) / 4);
  const int npl = (a.E + 63) / 64;
  if (npl <= 1)
    topk_kernel<1><<<grid, 256, 0, s>>>(a.logits, a.T, a.E, a.K, a.renorm, a.ids, a.w);
  else if (npl <= 2)
    topk_kernel<2><<<grid, 256, 0, s>>>(a.logits, a.T, a.E, a.K, a.renorm, a.ids, a.w);
  else if (npl <= 4)
    topk_kernel<4><<<grid, 256, 0, s>>>(a.logits, a.T, a.E, a.K, a.renorm, a.ids, a.w);
  else if (npl <= 8)
    topk_kernel<8><<<grid, 256, 0, s>>>(a.logits, a.T, a.E, a.K, a.renorm, a.ids, a.w);
  else
    topk_kernel<16><<<grid, 256, 0, s>>>(a.logits, a.T, a.E, a.K, a.renorm, a.ids, a.w);
  return hipGetLastError();
}

}  // namespace moe
