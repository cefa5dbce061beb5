/*
 * moe.h -- C ABI of the routed mixture-of-experts FFN layer for AMD MI355X
 * (gfx950).
 *
 * The layer (router softmax, top-k of E experts, SwiGLU experts with int8 or
 * int4 block-quantised weights, weighted combine plus an always-on shared
 * expert) is the MoE step of a Qwen3.6-35B-A3B-shaped model: 256 experts,
 * top-8 ("Qwen3.6-35B-A3B: pictures, several requests at once and speed",
 * introduction).  Its pieces follow the split the pages give the step: a
 * routing rule, the shared expert and the router's input, each invoked once
 * per layer and never from inside a kernel ("Models and backends", How a
 * backend works).
 *
 * Conventions for every entry point:
 *  - Pointers are DEVICE pointers owned by the caller unless marked "host".
 *    The library allocates no memory; all scratch lives in the caller's
 *    workspace `ws`.  No hidden staging buffers are shared between calls (a
 *    shared staging buffer silently corrupting an asynchronous expert group
 *    is the failure "qwen36: CUDA VRAM expert tier", Placement, describes).
 *  - Matrices are row-major with the reduction dimension contiguous; a weight
 *    matrix is [N][K_in].
 *  - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *    and the call returns without waiting; a device fault surfaces at the
 *    caller's next synchronisation.
 *  - A nonzero return means nothing was enqueued (argument errors) or a
 *    launch failed (MOE_ERR_HIP).  moe_status_string() describes a status.
 *  - Results are deterministic: identical inputs give identical bits on the
 *    same GPU and build, and on the decode path a token's output does not
 *    depend on which other tokens share the call.
 *  - Calls that share a workspace must be ordered on one stream.
 *
 * Weight formats (struct moe_experts):
 *  MOE_W_INT8_ROW  q int8 [E][N][K_in]; s float32 [E][N];  W = q * s[n].
 *  MOE_W_INT4_B32  q uint8 [E][N][K_in/2]; s binary16 [E][N][K_in/32];
 *                  byte j of a row holds element 2j in its low nibble and
 *                  2j+1 in its high nibble, each stored as q + 8 with q in
 *                  [-7, 7] (offset-binary nibbles: XOR with 8 gives the
 *                  two's-complement value, "Every Public GGUF of This Model
 *                  Is Missing Its Head", section 5); W = q * s[n][k/32].
 *                  A 16-byte aligned load is exactly one 32-element block.
 * Supported sizes: int4 hidden a multiple of 512 up to 4096 and ffn a
 * multiple of 512 up to 2048; int8 hidden a multiple of 256 up to 2048 and
 * ffn a multiple of 256 up to 1024; n_experts <= 1024;
 * top_k <= min(n_experts, 64).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* NULL pointer, bad size, inconsistent shapes */
  MOE_ERR_UNSUPPORTED = -2, /* valid but outside the supported sizes/formats */
  MOE_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required */
  MOE_ERR_HIP = -4          /* a HIP launch reported an error */
} moe_status;

typedef enum { MOE_W_INT8_ROW = 1, MOE_W_INT4_B32 = 2 } moe_wfmt;

/* A set of SwiGLU experts: gate/up are [E][ffn][hidden], down is
 * [E][hidden][ffn], in format `fmt`. */
typedef struct moe_experts {
  int32_t fmt;       /* moe_wfmt */
  int32_t n_experts; /* E for the routed set; 1 for a shared expert; 0 = absent */
  int32_t ffn;       /* SwiGLU width F */
  int32_t reserved;  /* must be 0 */
  const void *gate_q, *gate_s;
  const void *up_q, *up_s;
  const void *down_q, *down_s;
} moe_experts;

/* One MoE layer.  The router is float32 [E][hidden] (+ float32 [E] bias,
 * added to the logits before selection and softmax).  renorm = 1: the k
 * weights are a softmax over the k selected logits (softmax over all E then
 * renormalised); renorm = 0: the full softmax's values at the selected
 * experts.  shared_gate_w (float32 [hidden], 16-byte aligned, or NULL;
 * requires a shared expert): the shared expert's gate row.  Its product
 * with x is formed with the router's ("Qwen3.6-35B-A3B: pictures, several
 * requests at once and speed", Speed (0.1.45): the router and the shared
 * gate in one product) and the shared expert's output is scaled by its
 * sigmoid; NULL adds the shared expert with weight 1. */
typedef struct moe_layer {
  int32_t hidden;    /* H */
  int32_t n_experts; /* E */
  int32_t top_k;     /* K */
  int32_t renorm;
  const float *router_w;    /* [E][H] */
  const float *router_bias; /* [E] or NULL */
  moe_experts routed;       /* n_experts == E */
  moe_experts shared;       /* n_experts == 1, or 0 for no shared expert */
  const float *shared_gate_w; /* [H] or NULL */
} moe_layer;

/* Residual epilogue of a layer stack (host struct).  residual_out =
 * bf16_rne(residual_in + y); if normed_out is non-NULL it also receives
 * bf16_rne(r / sqrt(mean_h(r^2) + eps)) of r = residual_out, the
 * RMS-normalised input of the next layer (the pages' model normalises each
 * layer's input, "Qwen3.6-35B-A3B: pictures, several requests at once and
 * speed", Speed (0.1.45): add+norm in one launch).  residual_out may alias
 * residual_in and normed_out may alias the layer's own input x. */
typedef struct moe_residual {
  const uint16_t *residual_in; /* bf16 [T][H], required */
  uint16_t *residual_out;      /* bf16 [T][H], required */
  uint16_t *normed_out;        /* bf16 [T][H] or NULL */
  float eps;                   /* e.g. 1e-6 */
  int32_t reserved;            /* must be 0 */
} moe_residual;

/* Bytes of workspace moe_layer_forward needs for up to max_tokens tokens
 * (host, pure; 0 on invalid arguments). */
size_t moe_workspace_bytes(const moe_layer *L, int32_t max_tokens);

/* Prepares a workspace once before its first use (clears the control words
 * the kernels keep zero between calls).  Enqueued on `stream`. */
int moe_workspace_init(void *ws, size_t ws_bytes, void *stream);

/* Bytes of workspace moe_route needs for T tokens (host, pure; 0 on invalid
 * arguments): the logits when the caller passes none, plus, for batches of
 * more than 16 tokens, the router GEMM's partial sums. */
size_t moe_route_workspace_bytes(const moe_layer *L, int32_t T);

/* Router: logits[t][e] = sum_h Wr[e][h] * x[t][h] (+ bias[e]) in float32;
 * topk_ids[t][k] = the K largest logits in descending order, equal logits
 * going to the lower expert index (the pages' rule that the first of equal
 * largest values wins, "Models and backends", What was tuned);
 * topk_w[t][k] = routing weights per L->renorm.
 * x_bf16 [T][H] bfloat16 bits (16-byte aligned); topk_ids int32 [T][K];
 * topk_w float [T][K]; logits float [T][E], or NULL when the caller does not
 * want them.  ws (256-byte aligned, moe_route_workspace_bytes(L, T) bytes)
 * holds the logits when logits is NULL and, for batches of more than 16
 * tokens (whose logits are a matrix-core GEMM over slices of H, the slices
 * added in order by the top-k kernel), the partial sums; for a batch of at
 * most 16 tokens with logits given it is unused and may be NULL.
 * MOE_ERR_WORKSPACE if ws is needed and missing, misaligned or too small.  shared_gate float [T] or NULL: with L->shared_gate_w it
 * receives sigmoid(shared_gate_w . x[t]) per token. */
int moe_route(const moe_layer *L, const uint16_t *x_bf16, int32_t T, int32_t *topk_ids, float *topk_w,
              float *logits, float *shared_gate, void *ws, size_t ws_bytes, void *stream);

/* Workspace bytes moe_permute needs for T tokens, K slots, E experts. */
size_t moe_permute_workspace_bytes(int32_t T, int32_t K, int32_t E);

/* Token-by-expert permutation (the "grouping" that the pages move from a
 * host thread onto the card: "Qwen3.6-35B-A3B ...", Speed (0.1.45); "Strata
 * on an Intel Arc", Decode round 2).  Pair p = t*K + k goes to row
 * inv_pos[t][k]; rows are grouped by expert (ascending), and within an
 * expert ordered by p.  Outputs: counts int32 [E]; offsets int32 [E+1]
 * (exclusive prefix sum, offsets[E] = T*K); row_tok int32 [T*K] (token of
 * each row); row_w float [T*K] (topk_w of the pair, or 1 if topk_w is NULL);
 * inv_pos int32 [T][K]; active int32 [E] (experts with rows, ascending,
 * first *n_active entries valid); n_active int32 [1].  Integer results are
 * exact and deterministic. */
int moe_permute(const int32_t *topk_ids, const float *topk_w, int32_t T, int32_t K, int32_t E, int32_t *counts,
                int32_t *offsets, int32_t *row_tok, float *row_w, int32_t *inv_pos, int32_t *active,
                int32_t *n_active, void *ws, size_t ws_bytes, void *stream);

/* Workspace bytes moe_expert_ffn needs for n_rows rows of width ffn. */
size_t moe_expert_ffn_workspace_bytes(int32_t n_rows, int32_t ffn);

/* Expert FFN over permuted rows: for each row r of expert e (offsets[e] <=
 * r < offsets[e+1]), rows_out[r] = row_w[r] * D_e(silu(G_e x) * (U_e x))
 * with x = x_bf16[row_tok[r]].  Every expert's weights are read once for
 * all its rows ("Every Public GGUF of This Model Is Missing Its Head",
 * section 3: read the expert weights once per row group instead of per
 * token).  offsets/active/n_active as produced by moe_permute; when
 * W->n_experts == 1 they may be NULL (all n_rows rows belong to expert 0);
 * row_tok NULL means row r reads token r; row_w NULL means weight 1.
 * rows_out float [n_rows][hidden]. */
int moe_expert_ffn(const moe_experts *W, int32_t hidden, const uint16_t *x_bf16, int32_t T, int32_t n_rows,
                   const int32_t *offsets, const int32_t *active, const int32_t *n_active, const int32_t *row_tok,
                   const float *row_w, float *rows_out, void *ws, size_t ws_bytes, void *stream);

/* Combine, the MoE end of the layer: the weighted expert outputs plus the
 * shared expert's, summed per token ("Qwen3.6-35B-A3B: pictures, several
 * requests at once and speed", Speed (0.1.45): the MoE end in one launch of
 * 1024 threads, and add+norm of the residual in one launch; "Models and
 * backends", What was tuned: one launch adds up a call's experts).
 * y[t][h] = sum_{k<K} rows_out[inv_pos[t][k]][h] (k in order, each row
 * already scaled by its routing weight) + g[t] * shared_out[t][h] (one
 * fused multiply-add; g[t] = shared_gate[t], or 1 when shared_gate is
 * NULL); slots with inv_pos < 0 are skipped.  rows_out float [*][H]
 * (16-byte aligned); inv_pos int32 [T][K]; shared_out float [T][H] or NULL;
 * shared_gate float [T] or NULL; y float [T][H]; res (host) or NULL: the
 * residual epilogue above.  H a multiple of 256 up to 8192, K <= 64. */
int moe_combine(const float *rows_out, const int32_t *inv_pos, int32_t T, int32_t K, int32_t H,
                const float *shared_out, const float *shared_gate, float *y, const moe_residual *res, void *stream);

/* Stages of a layer call, for per-call profiling events. */
enum { MOE_STAGE_NONE = 0, MOE_STAGE_ROUTE = 1, MOE_STAGE_PERMUTE = 2, MOE_STAGE_GATEUP = 3,
       MOE_STAGE_DOWN = 4, MOE_STAGE_SHARED = 5, MOE_STAGE_COMBINE = 6, MOE_N_STAGES = 7 };

/* Kernel family of a layer call.  AUTO: the decode (GEMV-style) kernels for
 * T <= 16, the grouped-GEMM prefill kernels above.  DECODE / PREFILL force
 * one family at any T (the pages' practice of running one kernel family
 * beside another on the same activations to compare them, "Qwen3.6-35B-A3B:
 * pictures, several requests at once and speed", Speed (0.1.45)).  Both
 * families compute the same layer within the output tolerance; the prefill
 * family's range limits are stated at moe_layer_forward. */
typedef enum { MOE_PATH_AUTO = 0, MOE_PATH_DECODE = 1, MOE_PATH_PREFILL = 2 } moe_path;

/* Per-call options of moe_layer_forward_ex (host struct; all zero = the
 * defaults of moe_layer_forward). */
typedef struct moe_forward_opts {
  int32_t path;        /* moe_path */
  /* Tail-skip ("Models and backends", What was tuned: --tail-skip N): 0 =
   * off; N > 0: on a decode batch (T <= 16, not forced to the prefill
   * family) an expert that no token of the call ranks among its first N
   * picks is not computed, and the experts computed keep the weights the
   * router gave them (no renormalisation).  An approximation: it changes
   * the output.  Prompt batches are left untouched, as on the pages. */
  int32_t tail_skip;
  /* W8A8 variant: 0 = off; 1: the expert products take int8 activations
   * ("Strata on an Intel Arc", Arc Pro B70: the fused int8 expert path for
   * the prompt; "Models and backends", How each backend was checked: 8-bit
   * activations at every quantised matrix).  Every token's input and every
   * (token, expert) SwiGLU row is quantised with one symmetric scale per
   * row: amax = max |v|, q = round-half-even(v * (127 / amax)) in float32,
   * d = amax / 127; the int8 products accumulate exactly in int32 on the
   * int8 matrix cores and the row scales are applied once.  Needs int8
   * row-scaled weights (MOE_ERR_UNSUPPORTED otherwise; a shared expert must
   * be as wide as the routed ones) and changes the result by the
   * quantisation (about 1% of the output scale for N(0, 1) inputs). */
  int32_t act_quant;
  int32_t reserved; /* must be 0 */
  /* Profiling: hipEvent_t pairs (created by the caller) recorded on the
   * call's stream around each stage: index MOE_STAGE_*; a stage is profiled
   * when both of its events are non-NULL.  The gate/up and down stages'
   * kernels record their events at their own start and end (kernel time
   * without the launch gap); on calls of up to eight tokens the down
   * stage's kernel also does the combine, and the combine stage records
   * nothing. */
  void *stage_start[MOE_N_STAGES];
  void *stage_stop[MOE_N_STAGES];
} moe_forward_opts;

/* The whole layer: route, permute, routed experts, shared expert, combine
 * (the MoE step of "Qwen3.6-35B-A3B: pictures, several requests at once and
 * speed": 256 experts, top-8, a shared expert beside them; its Several
 * requests at once: the tokens of a batch share each expert's weight
 * reads).  y float [T][H]; res (host) or NULL: residual epilogue; topk_ids
 * [T][K] / topk_w [T][K] or NULL (copies of the routing used).  ws: at least
 * moe_workspace_bytes(L, T) bytes, 256-byte aligned, prepared once by
 * moe_workspace_init.  T = 0 is a no-op.
 *
 * Range of the prefill family (int4 weights, T > 16 or MOE_PATH_PREFILL):
 * its matrix products run in fp16, so every |x| must stay below 65504, every
 * dequantized weight |q * s| below 65504 and every SwiGLU value below 65504
 * in magnitude; a token outside that range gets non-finite outputs (other
 * tokens of the call are unaffected), where the decode family computes it
 * in fp32 and stays finite.  Values of a normalised layer input and of
 * block scales of real weights are many orders of magnitude inside it.
 *
 * The test-only environment variable MOE_FORCE_PATH=decode|prefill, read at
 * every call, forces the family of calls that leave the choice to AUTO. */
int moe_layer_forward(const moe_layer *L, const uint16_t *x_bf16, int32_t T, float *y, const moe_residual *res,
                      int32_t *topk_ids, float *topk_w, void *ws, size_t ws_bytes, void *stream);

/* moe_layer_forward with per-call options (opts NULL = defaults).
 * MOE_ERR_INVALID_ARG for an unknown path, a negative tail_skip or nonzero
 * reserved words. */
int moe_layer_forward_ex(const moe_layer *L, const uint16_t *x_bf16, int32_t T, float *y, const moe_residual *res,
                         int32_t *topk_ids, float *topk_w, void *ws, size_t ws_bytes, const moe_forward_opts *opts,
                         void *stream);

/* A stack of layers joined by the residual stream (the MoE steps of a
 * batch of requests passing through the model's layers one after another:
 * "Qwen3.6-35B-A3B: pictures, several requests at once and speed", Several
 * requests at once; "qwen36: CUDA VRAM expert tier", Placement: 40 layers of
 * 256 experts, top-8).  With x_0 = x_bf16 and r_0 = residual_in, for
 * l = 0 .. n_layers - 1:
 *   y = layer l applied to x_l (as moe_layer_forward),
 *   r_(l+1) = bf16(r_l + y), x_(l+1) = bf16(RMSNorm(r_(l+1))),
 * the residual epilogue of moe_residual with eps.  On return residual_out
 * holds r_n, normed_out x_n and y the last layer's y; topk_ids / topk_w (or
 * NULL) receive the last layer's routing.  Results are those of n_layers
 * moe_layer_forward calls chained the same way, up to the summation order
 * of the router products (each layer's combine also forms the next layer's
 * router product, so the routing launch of every layer after the first is
 * saved): selections agree except where two router logits are within
 * float32 rounding of each other.
 *
 * layers: n_layers >= 1 host structs of one shape (hidden, experts, top-k,
 * renorm, routed and shared formats and widths, shared gate present or
 * not), each valid for moe_layer_forward.  x_bf16, residual_in,
 * residual_out, normed_out: bf16 [T][H], 16-byte aligned; residual_in may
 * equal residual_out and x_bf16 may equal normed_out (the stack updates
 * them in place).  ws: moe_workspace_bytes(&layers[0], T) bytes as for
 * moe_layer_forward (it also holds a second residual buffer).  Errors are
 * those of moe_layer_forward, and MOE_ERR_INVALID_ARG for layers of
 * different shapes or missing residual buffers; on an error partway the
 * outputs hold an intermediate layer's state. */
int moe_stack_forward(const moe_layer *layers, int32_t n_layers, const uint16_t *x_bf16, int32_t T,
                      const uint16_t *residual_in, uint16_t *residual_out, uint16_t *normed_out, float eps, float *y,
                      int32_t *topk_ids, float *topk_w, void *ws, size_t ws_bytes, void *stream);

/* Bytes of the device array moe_layer_forward_noalloc uses as its
 * workspace (one array per GPU the library runs on). */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * moe_layer_forward_ex without a workspace argument.  The workspace is a
 * file-scope device array of MOE_NOALLOC_SCRATCH_BYTES bytes that each GPU
 * holds from the library's load until the process ends; the call itself
 * allocates nothing (no hipMalloc, hipFree or allocating library routine).
 * The first call on a device looks up that device's array address (with
 * the device current) and clears its control words on `stream`.
 * Arguments, results and errors are those of moe_layer_forward_ex, plus
 * MOE_ERR_UNSUPPORTED when the call needs more workspace than the array
 * holds (moe_workspace_bytes(L, T) > MOE_NOALLOC_SCRATCH_BYTES: e.g. about
 * 150 tokens of a 256-expert, H = 2048, top-8 layer) and MOE_ERR_HIP when
 * the array's address cannot be obtained.  Every call on one GPU shares
 * that GPU's array and leaves its contents behind: calls that overlap on
 * one GPU (other streams, other host threads) race and must be ordered by
 * the caller. */
int moe_layer_forward_noalloc(const moe_layer *L, const uint16_t *x_bf16, int32_t T, float *y,
                              const moe_residual *res, int32_t *topk_ids, float *topk_w,
                              const moe_forward_opts *opts, void *stream);

/* ---- Measurement helpers (not on the layer path) ----
 *
 * The achievable ceilings the expert kernels are compared with, measured on
 * the current device.  Each makes its launches on `stream` between two HIP
 * events it creates, waits for the second (host-blocking) and touches no
 * caller memory except what it is given to read.  Errors:
 * MOE_ERR_INVALID_ARG for arguments outside the stated ranges, MOE_ERR_HIP
 * for a failed launch or event. */

/* Matrix-core issue rate: 4 blocks a compute unit of 4 waves, each wave
 * issuing `iters` x 4 independent MFMAs from registers (no memory traffic):
 * kind 0 v_mfma_f32_32x32x16_f16, 1 v_mfma_f32_32x32x16_bf16,
 * 2 v_mfma_i32_32x32x32_i8.  One untimed launch precedes the timed one.
 * *ms receives the timed launch's duration and *ops the operations it
 * performed (2 per multiply-add).  1 <= iters <= 2^24. */
int moe_calib_mfma(int32_t kind, int32_t iters, float *ms, double *ops, void *stream);

/* HBM read rate: one launch that reads the `bytes` bytes at device address
 * `src` once (16-byte aligned, bytes a nonzero multiple of 16) with eight
 * 16-byte loads in flight per thread, at most one 1024-thread block a
 * compute unit.  *ms receives the launch's duration.  The rate is a ceiling
 * only when `src` is not already in the last-level cache: callers rotate
 * over buffers larger than it. */
int moe_calib_read(const void *src, size_t bytes, float *ms, void *stream);

/* Static text for a status code (host). */
const char *moe_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
