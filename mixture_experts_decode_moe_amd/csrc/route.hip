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
constexpr int kRouterExperts = 4;  // one expert per wave
constexpr int kRouterMaxChunks = 16;  // H <= 4096: 16-byte router chunks per lane

// One wave per expert row, one block per (4 experts, 16 tokens).  The token
// tile is staged in LDS once per block: every wave then reads its x values
// from LDS instead of all waves re-reading the same global lines.
__global__ void __launch_bounds__(256) router_logits_kernel(const float *__restrict__ wr,
                                                            const float *__restrict__ bias,
                                                            const uint16_t *__restrict__ x, int32_t T, int32_t H,
                                                            int32_t E, float *__restrict__ logits) {
  extern __shared__ uint2 xs[];  // [kRouterTokens][H/4] groups of four bf16
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int e = blockIdx.x * kRouterExperts + wave;
  const int t0 = blockIdx.y * kRouterTokens;
  const int nt = min(kRouterTokens, T - t0);
  const int h4 = H / 4;
  // this wave's router row first (all loads in flight at once), then the x
  // tile in batches of independent 16-byte loads
  const int nc = H / 256;  // <= kRouterMaxChunks
  float4 wv[kRouterMaxChunks];
  const float4 *wrow = reinterpret_cast<const float4 *>(wr + static_cast<size_t>(e < E ? e : 0) * H);
#pragma unroll
  for (int c = 0; c < kRouterMaxChunks; ++c)
    if (c < nc) wv[c] = wrow[c * 64 + lane];
  const int h8 = H / 8;
  const int n8 = nt * h8;
  for (int base = tid; base < n8; base += 256 * kStageBatch) {
    uint4 v[kStageBatch];
#pragma unroll
    for (int b = 0; b < kStageBatch; ++b) {
      const int i = base + 256 * b;
      if (i < n8) {
        const int t = i / h8, k = i - t * h8;
        v[b] = reinterpret_cast<const uint4 *>(x + static_cast<size_t>(t0 + t) * H)[k];
      }
    }
#pragma unroll
    for (int b = 0; b < kStageBatch; ++b) {
      const int i = base + 256 * b;
      if (i < n8) reinterpret_cast<uint4 *>(xs)[i] = v[b];
    }
  }
  __syncthreads();
  if (e >= E) return;
  float acc[kRouterTokens];
#pragma unroll
  for (int i = 0; i < kRouterTokens; ++i) acc[i] = 0.f;
#pragma unroll
  for (int c = 0; c < kRouterMaxChunks; ++c) {
    if (c >= nc) break;
#pragma unroll
    for (int i = 0; i < kRouterTokens; ++i) {
      if (i < nt) {
        const uint2 xv = xs[i * h4 + c * 64 + lane];
        acc[i] = fmaf(wv[c].x, bf16_lo(xv.x), acc[i]);
        acc[i] = fmaf(wv[c].y, bf16_hi(xv.x), acc[i]);
        acc[i] = fmaf(wv[c].z, bf16_lo(xv.y), acc[i]);
        acc[i] = fmaf(wv[c].w, bf16_hi(xv.y), acc[i]);
      }
    }
  }
  const float b = bias ? bias[e] : 0.f;
  float mine = 0.f;
#pragma unroll
  for (int i = 0; i < kRouterTokens; ++i) {
    if (i < nt) {
      const float s = sum64(acc[i]);
      if (lane == i) mine = s + b;
    }
  }
  if (lane < nt) logits[static_cast<size_t>(t0 + lane) * E + e] = mine;
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
MOE_DEV void key_max_step(uint32_t &hi, uint32_t &lo) {
  const uint32_t ph = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(hi), CTRL, 0xF, 0xF, true));
  const uint32_t pl = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(lo), CTRL, 0xF, 0xF, true));
  const bool take = (ph > hi) || (ph == hi && pl > lo);
  hi = take ? ph : hi;
  lo = take ? pl : lo;
}

MOE_DEV void key_take(uint32_t &hi, uint32_t &lo, uint32_t oh, uint32_t ol) {
  if (oh > hi || (oh == hi && ol > lo)) {
    hi = oh;
    lo = ol;
  }
}

// Wave-wide maximum of 64-bit keys (hi, lo); the result is uniform.
MOE_DEV void wave_key_max(uint32_t &hi, uint32_t &lo) {
  key_max_step<0xB1>(hi, lo);   // quad_perm [1,0,3,2]
  key_max_step<0x4E>(hi, lo);   // quad_perm [2,3,0,1]
  key_max_step<0x141>(hi, lo);  // row_half_mirror
  key_max_step<0x140>(hi, lo);  // row_mirror
  uint32_t bh = __builtin_amdgcn_readlane(hi, 0), bl = __builtin_amdgcn_readlane(lo, 0);
  key_take(bh, bl, __builtin_amdgcn_readlane(hi, 16), __builtin_amdgcn_readlane(lo, 16));
  key_take(bh, bl, __builtin_amdgcn_readlane(hi, 32), __builtin_amdgcn_readlane(lo, 32));
  key_take(bh, bl, __builtin_amdgcn_readlane(hi, 48), __builtin_amdgcn_readlane(lo, 48));
  hi = bh;
  lo = bl;
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
  uint32_t key[NPL];  // 0 = used or absent
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    const int e = lane + 64 * j;
    float val = -INFINITY;
    if (e < E) {
      val = l[e];
      if (val != val) val = -INFINITY;  // NaN never outranks a number
    }
    v[j] = val;
    key[j] = (e < E) ? float_key(val) : 0u;
  }
  float top_v = 0.f;
  float my_v = 0.f;  // lane k keeps round k's value and index
  int my_e = 0;
  for (int k = 0; k < K; ++k) {
    uint32_t hi = 0, lo = 0;
#pragma unroll
    for (int j = 0; j < NPL; ++j)
      key_take(hi, lo, key[j], key[j] ? 0xFFFFu - static_cast<uint32_t>(lane + 64 * j) : 0u);
    wave_key_max(hi, lo);
    const int sel_e = static_cast<int>(0xFFFFu - (lo & 0xFFFFu));
    const float sel_v = key_float(hi);
    if ((sel_e & 63) == lane) {
#pragma unroll
      for (int j = 0; j < NPL; ++j)
        if (lane + 64 * j == sel_e) key[j] = 0u;
    }
    if (k == 0) top_v = sel_v;
    if (lane == k) {
      my_v = sel_v;
      my_e = sel_e;
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
  if (lane < K) {
    ids[static_cast<size_t>(t) * K + lane] = my_e;
    wout[static_cast<size_t>(t) * K + lane] = mine / denom;
  }
}

hipError_t launch_router_logits(const RouteArgs &a, hipStream_t s) {
  dim3 grid((a.E + kRouterExperts - 1) / kRouterExperts, (a.T + kRouterTokens - 1) / kRouterTokens);
  const size_t lds = static_cast<size_t>(kRouterTokens) * a.H * 2;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&router_logits_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
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
