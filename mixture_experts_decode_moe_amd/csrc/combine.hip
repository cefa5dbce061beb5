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

// Chunk c (four elements) of token t's row: the routed rows in slot order
// (with K <= kCombineSlots every row is requested at once; the slot rows are
// block-uniform, read through the scalar cache), then the shared expert's
// row (scaled by its gate).  combine_load issues the chunk's loads;
// combine_finish writes y and, with residual_out, the residual sum
// r' = bf16(r + y), whose fp32 values go to r4 and squares into sq; `store`
// false computes without writing (the combine + router kernel's other
// blocks).  Split so that a caller can issue other loads between the two.
struct CombineLoads {
  float4 v[kCombineSlots];  // the slot rows (K <= kCombineSlots)
  float4 sv;                // the shared expert's row
  uint2 xv;                 // the residual
};

template <bool F16>
MOE_DEV void combine_load(const CombineArgs &a, int t, int c, CombineLoads &L) {
  const int n4 = a.H / 4;
  const int K = a.K;
  const int32_t *inv = a.inv_pos + static_cast<size_t>(t) * K;
  const size_t o4 = static_cast<size_t>(t) * n4 + c;
  if (K <= kCombineSlots) {
#pragma unroll
    for (int k = 0; k < kCombineSlots; ++k) {
      const int row = k < K ? inv[k] : -1;
      const float4 x = row4<F16>(a.rows_out, static_cast<size_t>(row < 0 ? 0 : row), a.H, c);
      L.v[k] = row >= 0 ? x : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  L.sv = a.shared_out ? row4<F16>(a.shared_out, static_cast<size_t>(t), a.H, c) : make_float4(0.f, 0.f, 0.f, 0.f);
  L.xv = a.residual_out ? reinterpret_cast<const uint2 *>(a.residual_in)[o4] : make_uint2(0u, 0u);
}

template <bool F16>
MOE_DEV void combine_finish(const CombineArgs &a, int t, int c, const CombineLoads &L, bool store, float4 &r4,
                            float &sq) {
  const int n4 = a.H / 4;
  const int K = a.K;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (K <= kCombineSlots) {
#pragma unroll
    for (int k = 0; k < kCombineSlots; ++k)
      if (k < K) add4(acc, L.v[k]);
  } else {
    const int32_t *inv = a.inv_pos + static_cast<size_t>(t) * K;
    for (int k = 0; k < K; ++k) {
      const int row = inv[k];
      if (row >= 0) add4(acc, row4<F16>(a.rows_out, static_cast<size_t>(row), a.H, c));
    }
  }
  const size_t o4 = static_cast<size_t>(t) * n4 + c;
  if (a.shared_out) {
    if (a.shared_gate) {
      // the shared expert's row scaled by its gate, fused into the sum
      const float g = a.shared_gate[t];
      acc.x = fmaf(g, L.sv.x, acc.x);
      acc.y = fmaf(g, L.sv.y, acc.y);
      acc.z = fmaf(g, L.sv.z, acc.z);
      acc.w = fmaf(g, L.sv.w, acc.w);
    } else {
      add4(acc, L.sv);
    }
  }
  if (store) reinterpret_cast<float4 *>(a.y)[o4] = acc;
  if (a.residual_out) {
    const uint16_t b0 = f32_to_bf16_rne(bf16_lo(L.xv.x) + acc.x);
    const uint16_t b1 = f32_to_bf16_rne(bf16_hi(L.xv.x) + acc.y);
    const uint16_t b2 = f32_to_bf16_rne(bf16_lo(L.xv.y) + acc.z);
    const uint16_t b3 = f32_to_bf16_rne(bf16_hi(L.xv.y) + acc.w);
    if (store)
      reinterpret_cast<uint2 *>(a.residual_out)[o4] =
          make_uint2(static_cast<uint32_t>(b0) | (static_cast<uint32_t>(b1) << 16),
                     static_cast<uint32_t>(b2) | (static_cast<uint32_t>(b3) << 16));
    r4 = make_float4(bf16_to_f32(b0), bf16_to_f32(b1), bf16_to_f32(b2), bf16_to_f32(b3));
    sq = fmaf(r4.x, r4.x, sq);
    sq = fmaf(r4.y, r4.y, sq);
    sq = fmaf(r4.z, r4.z, sq);
    sq = fmaf(r4.w, r4.w, sq);
  }
}

// 1 / sqrt(mean(r'^2) + eps) of the block's row: wave sums, then the waves
// in order (every thread of the block calls it).
MOE_DEV float row_inv_rms(float sq, float *wave_sq, int H, float eps) {
  sq = sum64(sq);
  if ((threadIdx.x & 63) == 0) wave_sq[threadIdx.x >> 6] = sq;
  lds_barrier();
  float total = 0.f;
#pragma unroll
  for (int w = 0; w < kCombineThreads / 64; ++w) total += wave_sq[w];
  return 1.f / sqrtf(total / static_cast<float>(H) + eps);
}

// bf16(r' * inv_rms) of four elements, packed.
MOE_DEV uint2 normed4(const float4 &r, float inv_rms) {
  const uint16_t b0 = f32_to_bf16_rne(r.x * inv_rms);
  const uint16_t b1 = f32_to_bf16_rne(r.y * inv_rms);
  const uint16_t b2 = f32_to_bf16_rne(r.z * inv_rms);
  const uint16_t b3 = f32_to_bf16_rne(r.w * inv_rms);
  return make_uint2(static_cast<uint32_t>(b0) | (static_cast<uint32_t>(b1) << 16),
                    static_cast<uint32_t>(b2) | (static_cast<uint32_t>(b3) << 16));
}

// One block per token row.  F16: the rows (and the shared expert's) are fp16.
template <bool F16>
__global__ void __launch_bounds__(kCombineThreads) combine_kernel(CombineArgs a) {
  __shared__ float wave_sq[kCombineThreads / 64];
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int n4 = a.H / 4;
  float4 r[kCombineChunks];
  float sq = 0.f;
#pragma unroll
  for (int i = 0; i < kCombineChunks; ++i) {
    const int c = tid + kCombineThreads * i;
    if (c >= n4) break;
    CombineLoads L;
    combine_load<F16>(a, t, c, L);
    combine_finish<F16>(a, t, c, L, true, r[i], sq);
  }
  if (!a.normed_out) return;
  const float inv_rms = row_inv_rms(sq, wave_sq, a.H, a.eps);
#pragma unroll
  for (int i = 0; i < kCombineChunks; ++i) {
    const int c = tid + kCombineThreads * i;
    if (c >= n4) break;
    reinterpret_cast<uint2 *>(a.normed_out)[static_cast<size_t>(t) * n4 + c] = normed4(r[i], inv_rms);
  }
}

// The last step of a stack layer fused with the first of the next: block
// (t, g) forms token t's combine, residual sum and normalised row exactly as
// combine_kernel does (group 0 writes them), then multiplies the normalised
// row by rows 16 g .. 16 g + 15 of the next layer's router product (the
// router rows, then the shared gate row as row E) and writes those products
// for the next layer's routing.  Each thread holds four columns (H <= 2048).
// The expert rows are requested first and the router rows after them, so
// the combine waits only for its own loads while the router rows arrive.
// A product is summed over a thread's four columns in order, then over the
// wave by a transposed reduction (lane halves exchange half of the sixteen
// sums, then 16-lane rows exchange half of the rest, then each 16-lane row
// adds its four sums), then over the waves in order.
constexpr int kCrRows = 16;

// The (token, group) pair of block b of the T x G blocks.  Block b runs on
// XCD b mod 8, and each XCD has its own L2: the pairs are laid out in bands
// of kCrBand tokens, group-major within a band, and each XCD takes a
// contiguous run of that order, so its blocks share the router rows of a few
// groups and the expert rows of a few tokens.  (With t fastest in the block
// id, every XCD held all groups and read the whole router matrix: eight
// copies of it from HBM a launch.)
constexpr int kCrBand = 8;

MOE_DEV void cr_pair(int b, int T, int G, int &t, int &g) {
  const int N = T * G, q = N >> 3, rem = N & 7, x = b & 7;
  const int p = x * q + (x < rem ? x : rem) + (b >> 3);  // blocks on XCDs < x come first
  const int full = T / kCrBand;
  const int nb = p < full * kCrBand * G ? kCrBand : T - kCrBand * full;  // tokens in p's band
  const int band = p / (kCrBand * G), r = p - band * kCrBand * G;
  g = r / nb;
  t = kCrBand * band + (r - g * nb);
}

__global__ void __launch_bounds__(kCombineThreads) combine_route_kernel(CombineRouteArgs a) {
  __shared__ float wave_sq[kCombineThreads / 64];
  __shared__ float wave_dot[kCombineThreads / 64][kCrRows];
  int t, g;
  cr_pair(blockIdx.x, a.c.T, (a.Ep + kCrRows - 1) / kCrRows, t, g);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const CombineArgs &c = a.c;
  const int n4 = c.H / 4;
  const bool mine = tid < n4;
  const int col = mine ? tid : 0;
  CombineLoads L;
  combine_load<false>(c, t, col, L);
  float4 wv[kCrRows];
#pragma unroll
  for (int j = 0; j < kCrRows; ++j) {
    const int row = g * kCrRows + j;
    const float *wr = row < a.E ? a.router_w + static_cast<size_t>(row) * c.H : a.gate_w;
    wv[j] = (mine && row < a.Ep) ? reinterpret_cast<const float4 *>(wr)[col] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float4 r4 = make_float4(0.f, 0.f, 0.f, 0.f);
  float sq = 0.f;
  if (mine) combine_finish<false>(c, t, col, L, g == 0, r4, sq);
  const float inv_rms = row_inv_rms(sq, wave_sq, c.H, c.eps);
  const uint2 nv = normed4(r4, inv_rms);
  if (mine && g == 0) reinterpret_cast<uint2 *>(c.normed_out)[static_cast<size_t>(t) * n4 + col] = nv;
  const float x0 = bf16_lo(nv.x), x1 = bf16_hi(nv.x), x2 = bf16_lo(nv.y), x3 = bf16_hi(nv.y);
  float d[kCrRows];
#pragma unroll
  for (int j = 0; j < kCrRows; ++j) {
    float v = wv[j].x * x0;
    v = fmaf(wv[j].y, x1, v);
    v = fmaf(wv[j].z, x2, v);
    v = fmaf(wv[j].w, x3, v);
    d[j] = mine ? v : 0.f;
  }
  // lane halves: afterwards d[j] (j < 8) is row j + 8 (lane / 32) over lanes l, l ^ 32
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(d[j]), __float_as_uint(d[8 + j]), false, false);
    d[j] = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  }
  // 16-lane rows: d[j] (j < 4) is row j + 4 ((lane / 16) % 2) + 8 (lane / 32) over four lanes
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(d[j]), __float_as_uint(d[4 + j]), false, false);
    d[j] = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) d[j] = sum16(d[j]);
  if ((lane & 15) == 0) {
    const int r0 = 4 * ((lane >> 4) & 1) + 8 * (lane >> 5);
#pragma unroll
    for (int j = 0; j < 4; ++j) wave_dot[wave][r0 + j] = d[j];
  }
  lds_barrier();
  if (tid < kCrRows) {
    const int row = g * kCrRows + tid;
    float total = 0.f;
#pragma unroll
    for (int w = 0; w < kCombineThreads / 64; ++w) total += wave_dot[w][tid];
    if (row < a.Ep) a.logits[static_cast<size_t>(t) * a.Ep + row] = total;
    if (a.sorted && g * kCrRows < a.E) {
      // the group's experts in selection order: the biased logit as the
      // routing forms it ((0 + product) + bias, NaN as -inf), ranked by
      // (key desc, expert asc) among the group's 16 rows; the first
      // kSortedKeep are written at their ranks
      const bool ex = row < a.E;
      const float v = (0.f + total) + (a.bias && ex ? a.bias[row] : 0.f);
      const uint32_t key = ex ? float_key(v == v ? v : -INFINITY) : 0u;
      int rank = 0;
#pragma unroll
      for (int j = 0; j < kCrRows; ++j) {
        const uint32_t kj = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(key), j));
        rank += (kj > key || (kj == key && j < tid)) ? 1 : 0;
      }
      if (rank < kSortedKeep)
        a.sorted[(static_cast<size_t>(t) * route_sorted_groups(a.E) + g) * kSortedKeep + rank] =
            make_uint2(key, static_cast<uint32_t>(row));
    }
  }
}

static_assert(kCrRows == kSortedGroup, "a block's router rows are one sorted group");

bool combine_route_ok(int H) { return H % 256 == 0 && H / 4 <= kCombineThreads; }

hipError_t launch_combine_route(const CombineRouteArgs &a, hipStream_t s) {
  if (a.c.T == 0) return hipSuccess;
  if (!combine_route_ok(a.c.H) || !a.c.normed_out || !a.c.residual_out) return hipErrorInvalidValue;
  const int blocks = a.c.T * ((a.Ep + kCrRows - 1) / kCrRows);
  combine_route_kernel<<<blocks, kCombineThreads, 0, s>>>(a);
  return hipGetLastError();
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
