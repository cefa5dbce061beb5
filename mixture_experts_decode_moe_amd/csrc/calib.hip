// Measurement helpers: the achievable ceilings that the expert kernels are
// compared with, measured on the device at hand rather than taken from the
// data sheet.
//
// - Matrix cores: a kernel that does nothing but issue independent 32x32
//   MFMAs from registers (four accumulators a wave, four blocks of four
//   waves a compute unit: four waves a SIMD), so its rate is the issue rate
//   of the matrix cores with no memory traffic and no vector work beside
//   it.  (Measured on one MI355X: 1.84 PFLOP/s fp16 with four waves a SIMD,
//   1.77 with two, 1.44-1.56 with one; eight accumulators a wave changed
//   little.)
// - HBM reads: a grid-stride kernel that streams a buffer once with eight
//   16-byte loads in flight per thread and keeps only an XOR of the data, the
//   read rate one launch of that size reaches.
//
// Both time themselves with HIP events on the caller's stream and wait for
// the stop event, so they are host-blocking; they touch no workspace.
#include <stdint.h>

#include "common.h"

namespace moe {

typedef uint32_t c_u32x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 c_f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 c_bf16x8_t __attribute__((ext_vector_type(8)));
typedef float c_f32x16_t __attribute__((ext_vector_type(16)));
typedef int c_i32x4_t __attribute__((ext_vector_type(4)));
typedef int c_i32x16_t __attribute__((ext_vector_type(16)));

constexpr int kCalibThreads = 256;

// KIND 0: v_mfma_f32_32x32x16_f16, 1: v_mfma_f32_32x32x16_bf16,
// 2: v_mfma_i32_32x32x32_i8.  Every iteration issues four MFMAs into four
// independent accumulators.
template <int KIND>
__global__ void __launch_bounds__(kCalibThreads) mfma_peak_kernel(int32_t iters, float *__restrict__ sink) {
  const uint32_t seed = threadIdx.x * 2654435761u + blockIdx.x;
  const c_u32x4_t bits = {seed, seed ^ 0x5bd1e995u, seed + 0x9e3779b9u, seed ^ 0x27d4eb2fu};
  // operands of small magnitude (exponent bits masked), so nothing overflows
  const c_u32x4_t small = {bits.x & 0x13FF13FFu, bits.y & 0x13FF13FFu, bits.z & 0x13FF13FFu, bits.w & 0x13FF13FFu};
  if constexpr (KIND == 2) {
    const c_i32x4_t a = __builtin_bit_cast(c_i32x4_t, bits & 0x03030303u);
    const c_i32x4_t b = __builtin_bit_cast(c_i32x4_t, (bits >> 8) & 0x03030303u);
    c_i32x16_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int i = 0; i < iters; ++i) {
      c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c3, 0, 0, 0);
    }
    int s = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) s ^= c0[j] ^ c1[j] ^ c2[j] ^ c3[j];
    if (s == 0x7fffffff) sink[blockIdx.x] = static_cast<float>(s);  // practically never: keeps the work
  } else {
    c_f32x16_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int i = 0; i < iters; ++i) {
      if constexpr (KIND == 0) {
        const c_f16x8_t a = __builtin_bit_cast(c_f16x8_t, small);
        const c_f16x8_t b = __builtin_bit_cast(c_f16x8_t, small ^ 0x00010001u);
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c3, 0, 0, 0);
      } else {
        const c_bf16x8_t a = __builtin_bit_cast(c_bf16x8_t, small);
        const c_bf16x8_t b = __builtin_bit_cast(c_bf16x8_t, small ^ 0x00010001u);
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
      }
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) s += c0[j] + c1[j] + c2[j] + c3[j];
    if (s == 12345.5f) sink[blockIdx.x] = s;  // practically never: keeps the work
  }
}

constexpr int kReadThreads = 1024;
constexpr int kReadInFlight = 8;

__global__ void __launch_bounds__(kReadThreads) read_stream_kernel(const uint4 *__restrict__ p, size_t n16,
                                                                    float *__restrict__ sink) {
  uint32_t acc = 0;
  const size_t stride = static_cast<size_t>(gridDim.x) * kReadThreads * kReadInFlight;
  for (size_t base = static_cast<size_t>(blockIdx.x) * kReadThreads * kReadInFlight + threadIdx.x; base < n16;
       base += stride) {
    uint4 v[kReadInFlight];
#pragma unroll
    for (int u = 0; u < kReadInFlight; ++u) {
      const size_t i = base + static_cast<size_t>(u) * kReadThreads;
      v[u] = i < n16 ? p[i] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kReadInFlight; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9e3779b9u) sink[blockIdx.x] = static_cast<float>(acc);  // practically never: keeps the loads
}

static __device__ float g_calib_sink[4096];

static int compute_units() {
  int dev = 0, v = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) return 256;
  return v;
}

// Times one launch made by `launch` between two events on stream s.
template <class Fn>
static int time_launch(hipStream_t s, float *ms, Fn launch) {
  hipEvent_t a = nullptr, b = nullptr;
  if (hipEventCreate(&a) != hipSuccess) return MOE_ERR_HIP;
  if (hipEventCreate(&b) != hipSuccess) {
    (void)hipEventDestroy(a);
    return MOE_ERR_HIP;
  }
  hipError_t e = hipEventRecord(a, s);
  if (e == hipSuccess) e = launch();
  if (e == hipSuccess) e = hipEventRecord(b, s);
  if (e == hipSuccess) e = hipEventSynchronize(b);
  if (e == hipSuccess) e = hipEventElapsedTime(ms, a, b);
  (void)hipEventDestroy(a);
  (void)hipEventDestroy(b);
  return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace moe

extern "C" {

int moe_calib_mfma(int32_t kind, int32_t iters, float *ms, double *ops, void *stream) {
  using namespace moe;
  if (kind < 0 || kind > 2 || iters <= 0 || iters > (1 << 24) || !ms || !ops) return MOE_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float *sink = nullptr;
  if (hipGetSymbolAddress(reinterpret_cast<void **>(&sink), HIP_SYMBOL(g_calib_sink)) != hipSuccess) return MOE_ERR_HIP;
  const int blocks = 4 * compute_units();
  if (blocks > 4096) return MOE_ERR_UNSUPPORTED;
  auto launch = [&]() {
    if (kind == 0)
      mfma_peak_kernel<0><<<blocks, kCalibThreads, 0, s>>>(iters, sink);
    else if (kind == 1)
      mfma_peak_kernel<1><<<blocks, kCalibThreads, 0, s>>>(iters, sink);
    else
      mfma_peak_kernel<2><<<blocks, kCalibThreads, 0, s>>>(iters, sink);
    return hipGetLastError();
  };
  // one untimed launch first (clocks, code load)
  if (launch() != hipSuccess) return MOE_ERR_HIP;
  const int rc = time_launch(s, ms, launch);
  if (rc != MOE_OK) return rc;
  // 32 x 32 outputs a wave, k = 16 (f16, bf16) or 32 (i8), two operations a product
  const double k = kind == 2 ? 32.0 : 16.0;
  *ops = 2.0 * 32 * 32 * k * 4.0 * iters * (kCalibThreads / 64) * blocks;
  return MOE_OK;
}

int moe_calib_read(const void *src, size_t bytes, float *ms, void *stream) {
  using namespace moe;
  if (!src || !ms || bytes == 0 || bytes % 16 || reinterpret_cast<uintptr_t>(src) % 16) return MOE_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float *sink = nullptr;
  if (hipGetSymbolAddress(reinterpret_cast<void **>(&sink), HIP_SYMBOL(g_calib_sink)) != hipSuccess) return MOE_ERR_HIP;
  const size_t n16 = bytes / 16;
  const size_t per_block = static_cast<size_t>(kReadThreads) * kReadInFlight;
  const size_t want = (n16 + per_block - 1) / per_block;
  const int cap = compute_units();
  const int blocks = static_cast<int>(want < static_cast<size_t>(cap) ? want : static_cast<size_t>(cap));
  return time_launch(s, ms, [&]() {
    read_stream_kernel<<<blocks, kReadThreads, 0, s>>>(static_cast<const uint4 *>(src), n16, sink);
    return hipGetLastError();
  });
}

}  // extern "C"
