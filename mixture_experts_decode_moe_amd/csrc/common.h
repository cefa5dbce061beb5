// Device helpers shared by the HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

#define MOE_DEV __device__ __forceinline__

namespace moe {

constexpr int kWave = 64;
constexpr int kStageBatch = 8;  // independent loads a thread issues before it stores them

// ---- bit-level conversions --------------------------------------------------

MOE_DEV float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
MOE_DEV float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }
MOE_DEV float bf16_to_f32(uint16_t b) { return __uint_as_float(static_cast<uint32_t>(b) << 16); }

// float32 -> bfloat16, round to nearest even: the chip's own conversion
// (v_cvt_pk_bf16_f32), two values an instruction when paired.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
MOE_DEV uint16_t f32_to_bf16_rne(float f) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f)); }
MOE_DEV uint32_t f32x2_to_bf16x2_rne(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

MOE_DEV float f16_bits_to_f32(uint16_t h) { return static_cast<float>(__builtin_bit_cast(_Float16, h)); }

// ---- DPP reductions ----------------------------------------------------------
// DPP controls (GFX9 encoding): quad_perm [1,0,3,2] = 0xB1, [2,3,0,1] = 0x4E,
// row_half_mirror = 0x141, row_mirror = 0x140.

template <int CTRL>
MOE_DEV float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Sum over each aligned group of 16 lanes; every lane of the group gets it.
MOE_DEV float sum16(float v) {
  v += dpp_f32<0xB1>(v);
  v += dpp_f32<0x4E>(v);
  v += dpp_f32<0x141>(v);
  v += dpp_f32<0x140>(v);
  return v;
}

// Sum over the wave in a fixed order ((row0 + row1) + (row2 + row3)); the
// result is uniform.
MOE_DEV float sum64(float v) {
  v = sum16(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (r0 + r1) + (r2 + r3);
}

MOE_DEV int lane_id() { return __lane_id(); }

// Order-preserving map of a float onto uint32 (NaN must be excluded).
MOE_DEV uint32_t float_key(float v) {
  const uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
MOE_DEV float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Block barrier for data exchanged through LDS only.  __syncthreads() also
// orders global memory at workgroup scope, which makes every wave wait for
// all its outstanding global loads and stores (prefetches included); this
// waits for the wave's LDS operations only.  The memory clobber keeps the
// compiler from moving memory accesses across it.
MOE_DEV void lds_barrier() { __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// ---- workspace carving -------------------------------------------------------

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

struct Carver {
  char *base;
  size_t off = 0;
  template <typename T>
  T *take(size_t count) {
    off = align_up(off, 256);
    T *p = base ? reinterpret_cast<T *>(base + off) : nullptr;
    off += count * sizeof(T);
    return p;
  }
};

// ---- launch helpers declared by each translation unit -----------------------

// Profiling events for one expert-kernel launch (both null when the call
// asks for none).
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};

// Which kernel family a call takes: chosen from the token count, or forced
// by the caller (moe_forward_opts::path).
enum PathSel : int32_t { kPathAuto = 0, kPathDecode = 1, kPathPrefill = 2 };

struct RouteArgs {
  const float *router_w;
  const float *router_bias;
  const uint16_t *x;
  int32_t T, H, E, K, renorm;
  float *logits;
  int32_t *ids;
  float *w;
  uint16_t *x16;  // optional [T][H]: x in fp16, pair-permuted 8-element pieces
  int32_t path;   // PathSel: kPathPrefill takes the matrix-core router GEMM at any T
  const float *gate_w;  // [H] or NULL: the shared expert's gate row
  float *gate;          // [T] (with gate_w): sigmoid of the gate row's product with x
  float *part;          // the router GEMM's partial sums: router_partial_floats(T, H, E, path) floats
};
hipError_t launch_router_logits(const RouteArgs &a, hipStream_t s);
// floats of partial sums the router GEMM needs for this call (0: the call
// takes the partial-logit router kernel and needs none)
size_t router_partial_floats(int T, int H, int E, int path);
// whether launch_router_logits writes x16 (when given) for this call
bool router_writes_x16(const RouteArgs &a);
hipError_t launch_topk(const RouteArgs &a, hipStream_t s);

// Router partial logits, then top-k + permutation in one block, for a decode
// batch.
constexpr int kFusedTokens = 16;    // largest T routed by the fused kernel
constexpr int kFusedMaxChunks = 2;  // router slice <= 512 floats: float4 per lane
// Decode routing from sorted expert groups.  The launch that forms a decode
// batch's whole router product (the previous stack layer's combine) can
// also write, for every token and every group of kSortedGroup experts, the
// group's first kSortedKeep (key, expert) pairs in selection order (larger
// biased logit first, the lower expert on equal logits, NaN as -inf; key =
// float_key of the logit, 0 for rows past E).  Every selected expert is
// among its group's first K, so with K <= kSortedKeep the gate/up kernel's
// routing merges these lists instead of ranking all E logits.  Taken only
// where the weights are a softmax over the K selected logits (renorm).
constexpr int kSortedGroup = 16;
constexpr int kSortedKeep = 8;
__host__ __device__ inline bool route_sorted_ok(int E, int K, int renorm) {
  return renorm == 1 && K >= 1 && K <= kSortedKeep && E >= K && E <= 256;
}
__host__ __device__ inline int route_sorted_groups(int E) { return (E + kSortedGroup - 1) / kSortedGroup; }

struct RouteFusedArgs {
  const float *router_w;
  const float *router_bias;
  const uint16_t *x;
  int32_t T, H, E, K, renorm;
  int32_t Hs, S;      // H slice per block and number of slices
  float *logits;      // [T][E] or NULL
  int32_t *ids;       // [T][K]
  float *w;           // [T][K]
  float *part;        // [S][T][Ep] partial logits (column E: the shared gate row's)
  int32_t *counts, *offsets, *row_tok, *inv_pos, *active, *n_active;
  float *row_w;
  int32_t *units;     // [E] int4 (expert, first row, rows, 0) per active unit, or NULL
  const float *gate_w;  // [H] or NULL: the shared expert's gate row, one more row of the product
  float *gate;          // [T] (with gate_w): sigmoid of the gate logit, published with the routing
  int32_t Ep;           // row stride of part: E, or E + 1 with the gate row
  int32_t tail_skip;    // 0, or N: experts no token ranks among its first N are left out
  const uint2 *sorted;  // [T][groups][kSortedKeep] (S = 1 only) or NULL: the logits' sorted groups
};
hipError_t launch_route_fused(const RouteFusedArgs &a, hipStream_t s);    // partials + selection
hipError_t launch_route_partial(const RouteFusedArgs &a, hipStream_t s);  // partials only
__host__ __device__ inline int route_fused_slice(int H) { return H % 512 == 0 ? 512 : 256; }

struct PermuteArgs {
  const int32_t *ids;
  const float *w;
  int32_t T, K, E;
  int32_t *counts, *offsets, *row_tok, *inv_pos, *active, *n_active;
  float *row_w;
  int32_t *tile_hist; // [n_tiles][E]
  int32_t *rank;      // [T*K]
};
constexpr int kPermuteTile = 1024;
hipError_t launch_permute(const PermuteArgs &a, hipStream_t s);

// Expert FFN over permuted rows (the GEMV path).  The routed units are the
// active experts (offsets != NULL) or a single expert 0 owning rows
// [0, n_rows) (offsets == NULL); when Fs > 0 the shared expert is one more
// unit whose rows t = 0..T-1 follow the routed rows in act and rows_out.
struct FfnArgs {
  int32_t fmt, H, F, Fs;
  const void *gq, *gs, *uq, *us, *dq, *ds;        // routed [E][..]
  const void *sgq, *sgs, *suq, *sus, *sdq, *sds;  // shared [1][..]
  const uint16_t *x;
  const uint16_t *x16;      // NULL, or x in fp16 as RouteArgs::x16 (prefill GEMMs read it)
  int32_t T;
  int32_t n_rows;           // routed rows
  int32_t n_experts;        // routed experts (offsets has n_experts + 1 entries)
  const int32_t *offsets;   // [E+1] or NULL
  const int32_t *active;    // [E]
  const int32_t *n_active;  // [1]
  const int32_t *row_tok;   // NULL: row r reads token r
  const float *row_w;       // NULL: weight 1
  float *act;               // [n_rows*F + T*Fs]
  float *rows_out;          // [n_rows + (Fs ? T : 0)][H], fp32 or (rows_f16) fp16
  int32_t rows_f16;         // 1: the down kernel writes rows_out in fp16 (prefill GEMM pair and W8A8 only)
  int32_t max_units;        // upper bound of routed units (grid sizing)
  const int32_t *units;     // [max_units] int4 (expert, first row, rows, 0) or NULL
  uint32_t *queue;          // NULL, or nine words, zero between calls: the prefill gate/up item queues
  // decode layer calls (E <= 256): the gate/up kernel routes the batch
  // itself from the router's partial logits and its last block publishes
  // the routing (the offsets, active, n_active, row_tok and row_w above
  // point at the same buffers for the kernels that follow)
  int32_t route_here;
  RouteFusedArgs route;
  int32_t path;          // PathSel
  int32_t distinct_ids;  // 1: every token picks an expert at most once, so a unit has at most T rows
  LaunchEvents ev;       // profiling events of the expert kernel of this stage (host side only)
  // W8A8 variant: x quantised per token [T][H] with scales [T]; the SwiGLU
  // rows (fp32 in act, F each) quantised per row [rows][F] with scales [rows]
  int8_t *qx;
  float *dx;
  int8_t *qa;
  float *da;
};
hipError_t launch_gateup(const FfnArgs &a, hipStream_t s);
bool mfma_decode_ok(const FfnArgs &a);  // the decode matrix-core kernels take this call
hipError_t launch_down(const FfnArgs &a, hipStream_t s);
// the prefill family's down launch for this call can write fp16 rows
// (rows_f16); the caller checks mfma_decode_ok first
bool down_rows_f16_ok(const FfnArgs &a);

// Down projection and combine in one launch (decode layer calls of a few
// tokens after the matrix-core gate/up kernel has published the routing).
struct DownCombineArgs {
  FfnArgs f;
  const int32_t *units;    // [max_units] int4 records (expert, first row, rows, 0)
  const int32_t *inv_pos;  // [T][K] permuted row of each slot
  int32_t K, E;
  float *y;                     // [T][H]
  const uint16_t *residual_in;  // with residual_out
  uint16_t *residual_out;       // NULL: no residual epilogue
  const float *shared_gate;     // [T] or NULL: the shared expert's row is scaled by it
};
bool down_combine_ok(const FfnArgs &a, int K);

// The W8A8 variant (int8 row-scaled weights, int8 activations): quantise x,
// gate/up + SwiGLU, quantise the SwiGLU rows, down x routing weight.
bool w8a8_ok(const FfnArgs &a);
hipError_t launch_w8a8(const FfnArgs &a, hipStream_t s, const LaunchEvents &ev_gu, const LaunchEvents &ev_dn);
hipError_t launch_down_combine(const DownCombineArgs &d, hipStream_t s);

struct CombineArgs {
  const float *rows_out;        // fp32 rows, or fp16 rows with rows_f16 (shared_out alike)
  const int32_t *inv_pos;
  int32_t T, K, H;
  const float *shared_out;      // [T][H] or NULL
  const float *shared_gate;     // [T] or NULL: shared_out's row t is scaled by it
  float *y;
  const uint16_t *residual_in;  // with residual_out
  uint16_t *residual_out;       // NULL: no residual epilogue
  uint16_t *normed_out;         // NULL: no normalised copy
  float eps;
  int32_t rows_f16;
};
hipError_t launch_combine(const CombineArgs &a, hipStream_t s);

// A stack layer's combine (with the residual sum and the normalised row)
// fused with the next layer's router product.
struct CombineRouteArgs {
  CombineArgs c;          // residual_out and normed_out required; fp32 rows
  const float *router_w;  // the next layer's router [E][H]
  const float *gate_w;    // its shared gate row [H], or NULL
  int32_t E, Ep;          // its experts; Ep = E (+ 1 with the gate row)
  float *logits;          // [T][Ep]: the next layer's router products (no bias)
  const float *bias;      // its router bias [E] or NULL (used for the sorted groups)
  uint2 *sorted;          // [T][groups][kSortedKeep] or NULL: the biased logits' sorted groups
};
bool combine_route_ok(int H);
hipError_t launch_combine_route(const CombineRouteArgs &a, hipStream_t s);

hipError_t launch_fill_zero(void *p, size_t bytes, hipStream_t s);

// Launches a kernel; with profiling events (a caller's per-call request)
// the runtime records them at the kernel's own start and end, so the
// interval is the kernel's execution time without the launch gap.
template <typename... KArgs, typename... Args>
hipError_t launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, uint32_t lds, hipStream_t s,
                         const LaunchEvents &ev, Args... args) {
  if (ev.start)
    hipExtLaunchKernelGGL(kernel, grid, block, lds, s, ev.start, ev.stop, 0u, args...);
  else
    kernel<<<grid, block, lds, s>>>(args...);
  return hipGetLastError();
}

}  // namespace moe
