// Combine ("the MoE end"): y[t] = sum over k of the routed rows of token t,
// in slot order, plus the shared expert's row; optionally the residual
// epilogue of a layer stack, r' = bf16(r + y) and the RMS-normalised
// bf16(r' / sqrt(mean(r'^2) + eps)) that feeds the next layer.  One launch
// sums every expert of the call ("Models and backends", What was tuned); a
// fixed summation order keeps the bits independent of scheduling.  One
// 512-thread block owns one token row, so the row's sum of squares is a
// block reduction in a fixed order.
#include <math.h>

#include "common.h"

namespace moe {

constexpr int kCombineThreads = 512;
constexpr int kCombineChunks = 4;  // float4 chunks per thread: H <= 8192
constexpr int kCombineSlots = 16;  // top-k slots summed from registers (K <= 16)

MOE_DEV void add4(float4 &a, const float4 &b) {
  a.x += b.x;
  a.y += b.y;
  a.z += b.z;
  a.w += b.w;
}

// Four consecutive elements of an expert row: fp32, or fp16 (F16).
template <bool F16>
MOE_DEV float4 row4(const float *rows, size_t row, int H, int c) {
  if constexpr (F16) {
    const uint2 v = reinterpret_cast<const uint2 *>(reinterpret_cast<const _Float16 *>(rows) + row * H)[c];
    typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
    const h2_t a = __builtin_bit_cast(h2_t, v.x), b = __builtin_bit_cast(h2_t, v.y);
    return make_float4(static_cast<float>(a[0]), static_cast<float>(a[1]), static_cast<float>(b[0]),
                       static_cast<float>(b[1]));
  } else {
    return reinterpret_cast<const float4 *>(rows + row * H)[c];
  }
}

// One block per token row.  With K <= kCombineSlots every row of a chunk is
// requested at once (the slot rows are block-uniform, read through the
// scalar cache), then added in slot order.  F16: the rows (and the shared
// expert's) are fp16.
template <bool F16>
__global__ void __launch_bounds__(kCombineThreads) combine_kernel(CombineArgs a) {
  __shared__ float wave_sq[kCombineThreads / 64];
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int n4 = a.H / 4;
  const int K = a.K;
  const int32_t *inv = a.inv_pos + static_cast<size_t>(t) * K;
  float4 r[kCombineChunks];
  float sq = 0.f;
#pragma unroll
  for (int i = 0; i < kCombineChunks; ++i) {
    const int c = tid + kCombineThreads * i;
    if (c >= n4) break;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (K <= kCombineSlots) {
      float4 v[kCombineSlots];
#pragma unroll
      for (int k = 0; k < kCombineSlots; ++k) {
        const int row = k < K ? inv[k] : -1;
        const float4 x = row4<F16>(a.rows_out, static_cast<size_t>(row < 0 ? 0 : row), a.H, c);
        v[k] = row >= 0 ? x : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int k = 0; k < kCombineSlots; ++k)
        if (k < K) add4(acc, v[k]);
    } else {
      for (int k = 0; k < K; ++k) {
        const int row = inv[k];
        if (row >= 0) add4(acc, row4<F16>(a.rows_out, static_cast<size_t>(row), a.H, c));
      }
    }
    const size_t o4 = static_cast<size_t>(t) * n4 + c;
    if (a.shared_out) {
      const float4 sv = row4<F16>(a.shared_out, static_cast<size_t>(t), a.H, c);
      if (a.shared_gate) {
        // the shared expert's row scaled by its gate, fused into the sum
        const float g = a.shared_gate[t];
        acc.x = fmaf(g, sv.x, acc.x);
        acc.y = fmaf(g, sv.y, acc.y);
        acc.z = fmaf(g, sv.z, acc.z);
        acc.w = fmaf(g, sv.w, acc.w);
      } else {
        add4(acc, sv);
      }
    }
    reinterpret_cast<float4 *>(a.y)[o4] = acc;
    if (a.residual_out) {
      const uint2 xv = reinterpret_cast<const uint2 *>(a.residual_in)[o4];
      const uint16_t b0 = f32_to_bf16_rne(bf16_lo(xv.x) + acc.x);
      const uint16_t b1 = f32_to_bf16_rne(bf16_hi(xv.x) + acc.y);
      const uint16_t b2 = f32_to_bf16_rne(bf16_lo(xv.y) + acc.z);
      const uint16_t b3 = f32_to_bf16_rne(bf16_hi(xv.y) + acc.w);
      reinterpret_cast<uint2 *>(a.residual_out)[o4] =
          make_uint2(static_cast<uint32_t>(b0) | (static_cast<uint32_t>(b1) << 16),
                     static_cast<uint32_t>(b2) | (static_cast<uint32_t>(b3) << 16));
      r[i] = make_float4(bf16_to_f32(b0), bf16_to_f32(b1), bf16_to_f32(b2), bf16_to_f32(b3));
      sq = fmaf(r[i].x, r[i].x, sq);
      sq = fmaf(r[i].y, r[i].y, sq);
      sq = fmaf(r[i].z, r[i].z, sq);
      sq = fmaf(r[i].w, r[i].w, sq);
    }
  }
  if (!a.normed_out) return;
  sq = sum64(sq);
  if ((tid & 63) == 0) wave_sq[tid >> 6] = sq;
  lds_barrier();
  float total = 0.f;
#pragma unroll
  for (int w = 0; w < kCombineThreads / 64; ++w) total += wave_sq[w];
  const float inv_rms = 1.f / sqrtf(total / static_cast<float>(a.H) + a.eps);
#pragma unroll
  for (int i = 0; i < kCombineChunks; ++i) {
    const int c = tid + kCombineThreads * i;
    if (c >= n4) break;
    const size_t o4 = static_cast<size_t>(t) * n4 + c;
    const uint16_t b0 = f32_to_bf16_rne(r[i].x * inv_rms);
    const uint16_t b1 = f32_to_bf16_rne(r[i].y * inv_rms);
    const uint16_t b2 = f32_to_bf16_rne(r[i].z * inv_rms);
    const uint16_t b3 = f32_to_bf16_rne(r[i].w * inv_rms);
    reinterpret_cast<uint2 *>(a.normed_out)[o4] =
        make_uint2(static_cast<uint32_t>(b0) | (static_cast<uint32_t>(b1) << 16),
                   static_cast<uint32_t>(b2) | (static_cast<uint32_t>(b3) << 16));
  }
}

hipError_t launch_combine(const CombineArgs &a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  if (a.rows_f16)
    combine_kernel<true><<<a.T, kCombineThreads, 0, s>>>(a);
  else
    combine_kernel<false><<<a.T, kCombineThreads, 0, s>>>(a);
  return hipGetLastError();
}

__global__ void fill_zero_kernel(uint32_t *p, size_t n) {
  for (size_t i = blockIdx.x * 256 + threadIdx.x; i < n; i += static_cast<size_t>(gridDim.x) * 256) p[i] = 0u;
}

hipError_t launch_fill_zero(void *p, size_t bytes, hipStream_t s) {
  const size_t n = bytes / 4;
  if (n == 0) return hipSuccess;
  const unsigned blocks = static_cast<unsigned>(n / 256 + 1 < 1024 ? n / 256 + 1 : 1024);
  fill_zero_kernel<<<blocks, 256, 0, s>>>(static_cast<uint32_t *>(p), n);
  return hipGetLastError();
}

}  // namespace moe
