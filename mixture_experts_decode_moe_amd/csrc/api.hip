// Host side of the C ABI declared in include/moe.h: argument validation,
// workspace carving and launch sequencing.  The library is stateless and
// allocates nothing; every buffer is the caller's.
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "common.h"

using namespace moe;

namespace {

hipStream_t as_stream(void *s) { return static_cast<hipStream_t>(s); }

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

int check_experts(const moe_experts &W, int32_t H, bool required_routed, int32_t E) {
  if (W.reserved != 0) return MOE_ERR_INVALID_ARG;
  if (W.n_experts == 0) return required_routed ? MOE_ERR_INVALID_ARG : MOE_OK;
  if (W.n_experts < 0) return MOE_ERR_INVALID_ARG;
  if (required_routed && W.n_experts != E) return MOE_ERR_INVALID_ARG;
  if (!required_routed && W.n_experts != 1) return MOE_ERR_INVALID_ARG;
  if (W.fmt != MOE_W_INT8_ROW && W.fmt != MOE_W_INT4_B32) return MOE_ERR_UNSUPPORTED;
  if (W.ffn <= 0) return MOE_ERR_INVALID_ARG;
  const void *ptrs[6] = {W.gate_q, W.gate_s, W.up_q, W.up_s, W.down_q, W.down_s};
  for (const void *p : ptrs)
    if (!p) return MOE_ERR_INVALID_ARG;
  if (!aligned(W.gate_q, 16) || !aligned(W.up_q, 16) || !aligned(W.down_q, 16)) return MOE_ERR_INVALID_ARG;
  if (!aligned(W.gate_s, 4) || !aligned(W.up_s, 4) || !aligned(W.down_s, 4)) return MOE_ERR_INVALID_ARG;
  if (W.fmt == MOE_W_INT4_B32) {
    if (H % 512 || W.ffn % 512 || H > 4096 || W.ffn > 2048) return MOE_ERR_UNSUPPORTED;
  } else {
    if (H % 256 || W.ffn % 256 || H > 2048 || W.ffn > 1024) return MOE_ERR_UNSUPPORTED;
  }
  return MOE_OK;
}

int check_layer(const moe_layer *L) {
  if (!L) return MOE_ERR_INVALID_ARG;
  if (L->hidden <= 0 || L->n_experts <= 0 || L->top_k <= 0) return MOE_ERR_INVALID_ARG;
  if (L->top_k > L->n_experts) return MOE_ERR_INVALID_ARG;
  if (L->n_experts > 1024 || L->top_k > 64) return MOE_ERR_UNSUPPORTED;
  if (L->renorm != 0 && L->renorm != 1) return MOE_ERR_INVALID_ARG;
  if (L->hidden % 256) return MOE_ERR_UNSUPPORTED;
  if (!L->router_w || !aligned(L->router_w, 16)) return MOE_ERR_INVALID_ARG;
  int rc = check_experts(L->routed, L->hidden, true, L->n_experts);
  if (rc != MOE_OK) return rc;
  rc = check_experts(L->shared, L->hidden, false, 1);
  if (rc != MOE_OK) return rc;
  // a gate row needs the shared expert it gates, and whole 16-byte rows
  if (L->shared_gate_w && (L->shared.n_experts != 1 || !aligned(L->shared_gate_w, 16))) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

// Partial-logit rows of the decode routing: the experts, plus the shared
// gate row when there is one.
int32_t router_rows(const moe_layer *L) { return L->n_experts + (L->shared_gate_w ? 1 : 0); }

// Where a stack layer's fused combine + router launch leaves the next
// layer's sorted expert groups for a T-token decode batch: after the whole
// router product [T][Ep] in the partial-logit area (S slices of it), when
// the next layer's routing can merge them and they fit; else NULL.
uint2 *sorted_groups(const moe_layer *N, float *part, int32_t T) {
  const int32_t E = N->n_experts, Ep = router_rows(N);
  if (!route_sorted_ok(E, N->top_k, N->renorm) || T > kFusedTokens) return nullptr;
  const int32_t S = N->hidden / route_fused_slice(N->hidden);
  const size_t logit_floats = (static_cast<size_t>(T) * Ep + 3) & ~static_cast<size_t>(3);  // 16-byte aligned after
  const size_t need = logit_floats + static_cast<size_t>(T) * route_sorted_groups(E) * kSortedKeep * 2;
  if (need > static_cast<size_t>(S) * T * Ep) return nullptr;
  return reinterpret_cast<uint2 *>(part + logit_floats);
}

constexpr size_t kControlBytes = 256;  // control words kept zero between calls

// The profiling events a call asked for (moe_forward_opts), one pair per
// stage.  A stage's expert kernel records its pair itself at its own start
// and end (launch_kernel); other stages are bracketed here.
struct CallEvents {
  hipEvent_t start[MOE_N_STAGES] = {}, stop[MOE_N_STAGES] = {};
  LaunchEvents of(int32_t st) const { return LaunchEvents{start[st], stop[st]}; }
};

// Records a stage's start event on construction and its stop event on
// destruction, unless the stage's expert kernel took the pair
// (kernel_takes = true).
struct StageMark {
  const CallEvents &ev;
  int32_t stage;
  hipStream_t s;
  bool kernel_takes;
  StageMark(const CallEvents &e, int32_t st, hipStream_t str, bool kernel = false)
      : ev(e), stage(st), s(str), kernel_takes(kernel) {
    if (!kernel_takes && ev.start[stage]) (void)hipEventRecord(ev.start[stage], s);
  }
  ~StageMark() {
    if (!kernel_takes && ev.stop[stage]) (void)hipEventRecord(ev.stop[stage], s);
  }
};

// The kernel family a call takes: the caller's choice, else the test-only
// override MOE_FORCE_PATH=decode|prefill (read at every call, so a process
// can switch it), else chosen from the token count.
int32_t effective_path(const moe_forward_opts *opts) {
  if (opts && opts->path != MOE_PATH_AUTO) return opts->path;
  const char *env = getenv("MOE_FORCE_PATH");
  if (env) {
    if (strcmp(env, "decode") == 0) return MOE_PATH_DECODE;
    if (strcmp(env, "prefill") == 0) return MOE_PATH_PREFILL;
  }
  return MOE_PATH_AUTO;
}

struct LayerWs {
  uint32_t *control;  // kControlBytes of words kept zero between calls; [0..8]: prefill gate/up item queues
  float *part;        // fused routing: partial logits [S][T][E]
  float *logits;
  int32_t *ids;
  float *w;
  int32_t *counts, *offsets, *active, *n_active, *row_tok, *inv_pos, *rank, *tile_hist;
  int32_t *units;  // [E][4]: expert, first row, rows, 0 of each active unit
  float *row_w;
  float *act, *rows_out;
  uint16_t *x16;  // x in fp16 for the prefill GEMMs, written by the router GEMM
  float *gate;    // [T]: the shared expert's gate values
  int8_t *qx, *qa;  // W8A8: quantised x [T][H] and SwiGLU rows [rows][F]
  float *dx, *da;   // their per-row scales
  float *rpart;     // the router GEMM's partial sums
  uint16_t *rstack;  // [T][H] bf16: the other residual buffer of a stack call
  size_t bytes;
};

LayerWs carve_layer(const moe_layer *L, int32_t T, void *base) {
  Carver c{static_cast<char *>(base)};
  LayerWs w{};
  w.control = c.take<uint32_t>(kControlBytes / 4);
  const size_t TK = static_cast<size_t>(T) * L->top_k;
  const size_t E = L->n_experts;
  const size_t n_tiles = (TK + kPermuteTile - 1) / kPermuteTile;
  const size_t S = static_cast<size_t>(L->hidden / route_fused_slice(L->hidden));
  // sized for min(T, kFusedTokens) tokens so that the total grows with T
  w.part = c.take<float>(S * static_cast<size_t>(T < kFusedTokens ? T : kFusedTokens) * router_rows(L));
  w.logits = c.take<float>(static_cast<size_t>(T) * E);
  w.ids = c.take<int32_t>(TK);
  w.w = c.take<float>(TK);
  w.counts = c.take<int32_t>(E);
  w.offsets = c.take<int32_t>(E + 1);
  w.active = c.take<int32_t>(E);
  w.n_active = c.take<int32_t>(1);
  w.row_tok = c.take<int32_t>(TK);
  w.row_w = c.take<float>(TK);
  w.inv_pos = c.take<int32_t>(TK);
  w.rank = c.take<int32_t>(TK);
  w.tile_hist = c.take<int32_t>(n_tiles * E);
  w.units = c.take<int32_t>(4 * E);
  // SwiGLU rows and expert output rows: the routed rows, then (with a shared
  // expert) its T rows
  const size_t Fs = L->shared.n_experts == 1 ? L->shared.ffn : 0;
  w.act = c.take<float>(TK * L->routed.ffn + static_cast<size_t>(T) * Fs);
  w.rows_out = c.take<float>((TK + (Fs ? T : 0)) * L->hidden);
  w.x16 = c.take<uint16_t>(static_cast<size_t>(T) * L->hidden);
  w.gate = c.take<float>(T);
  w.qx = c.take<int8_t>(static_cast<size_t>(T) * L->hidden);
  w.dx = c.take<float>(T);
  w.qa = c.take<int8_t>((TK + (Fs ? T : 0)) * L->routed.ffn);
  w.da = c.take<float>(TK + (Fs ? T : 0));
  // the router GEMM's partial sums of a prompt batch (either path may be
  // forced at run time, so sized for the GEMM whenever T allows it)
  w.rpart = c.take<float>(router_partial_floats(T, L->hidden, static_cast<int>(E), kPathPrefill));
  w.rstack = c.take<uint16_t>(static_cast<size_t>(T) * L->hidden);
  w.bytes = align_up(c.off, 256);
  return w;
}

FfnArgs ffn_args(const moe_experts &W, const moe_experts *S, int32_t H, const uint16_t *x, int32_t T,
                 int32_t n_rows) {
  FfnArgs a{};
  a.fmt = W.fmt;
  a.H = H;
  a.F = W.ffn;
  a.Fs = S ? S->ffn : 0;
  a.gq = W.gate_q;
  a.gs = W.gate_s;
  a.uq = W.up_q;
  a.us = W.up_s;
  a.dq = W.down_q;
  a.ds = W.down_s;
  if (S) {
    a.sgq = S->gate_q;
    a.sgs = S->gate_s;
    a.suq = S->up_q;
    a.sus = S->up_s;
    a.sdq = S->down_q;
    a.sds = S->down_s;
  }
  a.x = x;
  a.T = T;
  a.n_rows = n_rows;
  a.n_experts = W.n_experts;
  return a;
}

}  // namespace

extern "C" {

const char *moe_status_string(int status) {
  switch (status) {
    case MOE_OK:
      return "ok";
    case MOE_ERR_INVALID_ARG:
      return "invalid argument";
    case MOE_ERR_UNSUPPORTED:
      return "unsupported size or format";
    case MOE_ERR_WORKSPACE:
      return "workspace missing or too small";
    case MOE_ERR_HIP:
      return "HIP launch error";
    default:
      return "unknown status";
  }
}

size_t moe_workspace_bytes(const moe_layer *L, int32_t max_tokens) {
  if (check_layer(L) != MOE_OK || max_tokens < 0) return 0;
  return carve_layer(L, max_tokens, nullptr).bytes;
}

int moe_workspace_init(void *ws, size_t ws_bytes, void *stream) {
  if (!ws || ws_bytes < kControlBytes || !aligned(ws, 256)) return MOE_ERR_WORKSPACE;
  return hip_status(launch_fill_zero(ws, kControlBytes, as_stream(stream)));
}

size_t moe_route_workspace_bytes(const moe_layer *L, int32_t T) {
  if (check_layer(L) != MOE_OK || T < 0) return 0;
  // the logits (when the caller passes none), then the router GEMM's
  // partial sums (batches above kFusedTokens tokens)
  return align_up(static_cast<size_t>(T) * L->n_experts * sizeof(float), 256) +
         align_up(router_partial_floats(T, L->hidden, L->n_experts, kPathAuto) * sizeof(float), 256);
}

int moe_route(const moe_layer *L, const uint16_t *x_bf16, int32_t T, int32_t *topk_ids, float *topk_w, float *logits,
              float *shared_gate, void *ws, size_t ws_bytes, void *stream) {
  int rc = check_layer(L);
  if (rc != MOE_OK) return rc;
  if (T < 0) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!x_bf16 || !topk_ids || !topk_w || !aligned(x_bf16, 16)) return MOE_ERR_INVALID_ARG;
  // the workspace: the logits when the caller passes none, then the router
  // GEMM's partial sums when the batch takes the GEMM
  const size_t logit_bytes = align_up(static_cast<size_t>(T) * L->n_experts * sizeof(float), 256);
  const size_t part_floats = router_partial_floats(T, L->hidden, L->n_experts, kPathAuto);
  if (!logits || part_floats) {
    if (!ws || !aligned(ws, 256) || ws_bytes < moe_route_workspace_bytes(L, T)) return MOE_ERR_WORKSPACE;
    if (!logits) logits = static_cast<float *>(ws);
  }
  float *part = part_floats ? reinterpret_cast<float *>(static_cast<char *>(ws) + logit_bytes) : nullptr;
  const bool gate = L->shared_gate_w && shared_gate;
  RouteArgs a{L->router_w, L->router_bias, x_bf16, T, L->hidden, L->n_experts, L->top_k, L->renorm, logits,
              topk_ids, topk_w, nullptr, kPathAuto, gate ? L->shared_gate_w : nullptr, gate ? shared_gate : nullptr,
              part};
  hipError_t e = launch_router_logits(a, as_stream(stream));
  if (e == hipSuccess) e = launch_topk(a, as_stream(stream));
  return hip_status(e);
}

size_t moe_permute_workspace_bytes(int32_t T, int32_t K, int32_t E) {
  if (T < 0 || K <= 0 || E <= 0) return 0;
  const size_t TK = static_cast<size_t>(T) * K;
  const size_t n_tiles = (TK + kPermuteTile - 1) / kPermuteTile;
  Carver c{nullptr};
  c.take<int32_t>(TK);
  c.take<int32_t>(n_tiles * E);
  return align_up(c.off, 256);
}

int moe_permute(const int32_t *topk_ids, const float *topk_w, int32_t T, int32_t K, int32_t E, int32_t *counts,
                int32_t *offsets, int32_t *row_tok, float *row_w, int32_t *inv_pos, int32_t *active,
                int32_t *n_active, void *ws, size_t ws_bytes, void *stream) {
  if (T < 0 || K <= 0 || E <= 0 || K > E) return MOE_ERR_INVALID_ARG;
  if (E > 1024) return MOE_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(T) * K > INT32_MAX / 2) return MOE_ERR_UNSUPPORTED;
  if (!counts || !offsets || !active || !n_active) return MOE_ERR_INVALID_ARG;
  if (T > 0 && (!topk_ids || !row_tok || !row_w || !inv_pos)) return MOE_ERR_INVALID_ARG;
  const size_t need = moe_permute_workspace_bytes(T, K, E);
  if (!ws || ws_bytes < need) return MOE_ERR_WORKSPACE;
  Carver c{static_cast<char *>(ws)};
  const size_t TK = static_cast<size_t>(T) * K;
  PermuteArgs a{};
  a.ids = topk_ids;
  a.w = topk_w;
  a.T = T;
  a.K = K;
  a.E = E;
  a.counts = counts;
  a.offsets = offsets;
  a.row_tok = row_tok;
  a.row_w = row_w;
  a.inv_pos = inv_pos;
  a.active = active;
  a.n_active = n_active;
  a.rank = c.take<int32_t>(TK);
  a.tile_hist = c.take<int32_t>((TK + kPermuteTile - 1) / kPermuteTile * E);
  if (T == 0) {
    // No pairs: zero counts/offsets/n_active through the scatter kernel's
    // tile-0 path is unavailable (no tiles), so clear them directly.
    hipError_t e = launch_fill_zero(counts, static_cast<size_t>(E) * 4, as_stream(stream));
    if (e == hipSuccess) e = launch_fill_zero(offsets, static_cast<size_t>(E + 1) * 4, as_stream(stream));
    if (e == hipSuccess) e = launch_fill_zero(n_active, 4, as_stream(stream));
    return hip_status(e);
  }
  return hip_status(launch_permute(a, as_stream(stream)));
}

size_t moe_expert_ffn_workspace_bytes(int32_t n_rows, int32_t ffn) {
  if (n_rows < 0 || ffn <= 0) return 0;
  return align_up(static_cast<size_t>(n_rows) * ffn * sizeof(float), 256);
}

int moe_expert_ffn(const moe_experts *W, int32_t hidden, const uint16_t *x_bf16, int32_t T, int32_t n_rows,
                   const int32_t *offsets, const int32_t *active, const int32_t *n_active, const int32_t *row_tok,
                   const float *row_w, float *rows_out, void *ws, size_t ws_bytes, void *stream) {
  if (!W || hidden <= 0 || T < 0 || n_rows < 0) return MOE_ERR_INVALID_ARG;
  int rc = check_experts(*W, hidden, W->n_experts != 1, W->n_experts);
  if (rc != MOE_OK) return rc;
  if (W->n_experts == 0) return MOE_ERR_INVALID_ARG;
  if (W->n_experts > 1 && (!offsets || !active || !n_active)) return MOE_ERR_INVALID_ARG;
  if (!row_tok && n_rows > T) return MOE_ERR_INVALID_ARG;
  if (n_rows == 0) return MOE_OK;
  if (!x_bf16 || !rows_out || !aligned(x_bf16, 16) || !aligned(rows_out, 16)) return MOE_ERR_INVALID_ARG;
  if (!ws || ws_bytes < moe_expert_ffn_workspace_bytes(n_rows, W->ffn)) return MOE_ERR_WORKSPACE;
  FfnArgs a = ffn_args(*W, nullptr, hidden, x_bf16, T, n_rows);
  a.offsets = offsets;
  a.active = offsets ? active : nullptr;
  a.n_active = offsets ? n_active : nullptr;
  a.row_tok = row_tok;
  a.row_w = row_w;
  a.act = static_cast<float *>(ws);
  a.rows_out = rows_out;
  a.max_units = offsets ? (n_rows < W->n_experts ? n_rows : W->n_experts) : 1;
  hipError_t e = launch_gateup(a, as_stream(stream));
  if (e == hipSuccess) e = launch_down(a, as_stream(stream));
  return hip_status(e);
}

namespace {
int check_residual(const moe_residual *res, int32_t H) {
  if (!res) return MOE_OK;
  if (res->reserved != 0 || !res->residual_in || !res->residual_out) return MOE_ERR_INVALID_ARG;
  if (!aligned(res->residual_in, 8) || !aligned(res->residual_out, 8) ||
      (res->normed_out && !aligned(res->normed_out, 8)))
    return MOE_ERR_INVALID_ARG;
  if (!(res->eps >= 0.f)) return MOE_ERR_INVALID_ARG;
  (void)H;
  return MOE_OK;
}

CombineArgs combine_args(const float *rows_out, const int32_t *inv_pos, int32_t T, int32_t K, int32_t H,
                         const float *shared_out, const float *shared_gate, float *y, const moe_residual *res) {
  CombineArgs a{rows_out, inv_pos, T, K, H, shared_out, shared_out ? shared_gate : nullptr, y, nullptr, nullptr,
                nullptr, 0.f};
  if (res) {
    a.residual_in = res->residual_in;
    a.residual_out = res->residual_out;
    a.normed_out = res->normed_out;
    a.eps = res->eps;
  }
  return a;
}
}  // namespace

int moe_combine(const float *rows_out, const int32_t *inv_pos, int32_t T, int32_t K, int32_t H,
                const float *shared_out, const float *shared_gate, float *y, const moe_residual *res, void *stream) {
  if (T < 0 || K <= 0 || H <= 0 || H % 256 || H > 8192) return MOE_ERR_INVALID_ARG;
  if (K > 64) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!rows_out || !inv_pos || !y) return MOE_ERR_INVALID_ARG;
  if (!aligned(rows_out, 16) || !aligned(y, 16) || (shared_out && !aligned(shared_out, 16)))
    return MOE_ERR_INVALID_ARG;
  int rc = check_residual(res, H);
  if (rc != MOE_OK) return rc;
  return hip_status(
      launch_combine(combine_args(rows_out, inv_pos, T, K, H, shared_out, shared_gate, y, res), as_stream(stream)));
}

namespace {

// How a layer call of moe_stack_forward links to its neighbours: its router
// product is already in the workspace (written by the previous call's
// combine), and/or its combine also forms the next layer's router product.
struct StackLink {
  bool route_ready = false;
  const moe_layer *next = nullptr;
  bool *fused = nullptr;  // set when the call did form the next layer's product
};

int layer_forward(const moe_layer *L, const uint16_t *x_bf16, int32_t T, float *y, const moe_residual *res,
                  int32_t *topk_ids, float *topk_w, void *ws, size_t ws_bytes, const moe_forward_opts *opts,
                  void *stream, const StackLink &link) {
  if (link.fused) *link.fused = false;
  int rc = check_layer(L);
  if (rc != MOE_OK) return rc;
  if (T < 0) return MOE_ERR_INVALID_ARG;
  if (opts) {
    if (opts->path < MOE_PATH_AUTO || opts->path > MOE_PATH_PREFILL || opts->tail_skip < 0 ||
        (opts->act_quant != 0 && opts->act_quant != 1))
      return MOE_ERR_INVALID_ARG;
    // the W8A8 variant takes int8 row-scaled weights (and a shared expert as
    // wide as the routed ones)
    if (opts->act_quant &&
        (L->routed.fmt != MOE_W_INT8_ROW || (L->shared.n_experts == 1 && (L->shared.fmt != MOE_W_INT8_ROW ||
                                                                          L->shared.ffn != L->routed.ffn))))
      return MOE_ERR_UNSUPPORTED;
    if (opts->reserved != 0) return MOE_ERR_INVALID_ARG;
  }
  if (T == 0) return MOE_OK;
  if (static_cast<int64_t>(T) * L->top_k > INT32_MAX / 2) return MOE_ERR_UNSUPPORTED;
  if (!x_bf16 || !y || !aligned(x_bf16, 16) || !aligned(y, 16)) return MOE_ERR_INVALID_ARG;
  rc = check_residual(res, L->hidden);
  if (rc != MOE_OK) return rc;
  if (!ws || !aligned(ws, 256)) return MOE_ERR_WORKSPACE;
  LayerWs w = carve_layer(L, T, ws);
  if (ws_bytes < w.bytes) return MOE_ERR_WORKSPACE;
  hipStream_t s = as_stream(stream);
  const int32_t K = L->top_k, E = L->n_experts, H = L->hidden;
  int32_t *ids = topk_ids ? topk_ids : w.ids;
  float *tw = topk_w ? topk_w : w.w;
  const int32_t path = effective_path(opts);
  CallEvents ev;
  if (opts)
    for (int st = 1; st < MOE_N_STAGES; ++st) {
      // a stage is profiled only with both of its events
      if (opts->stage_start[st] && opts->stage_stop[st]) {
        ev.start[st] = static_cast<hipEvent_t>(opts->stage_start[st]);
        ev.stop[st] = static_cast<hipEvent_t>(opts->stage_stop[st]);
      }
    }

  const int32_t TK = T * K;
  const bool has_shared = L->shared.n_experts == 1;
  FfnArgs xa = ffn_args(L->routed, has_shared ? &L->shared : nullptr, H, x_bf16, T, TK);
  xa.offsets = w.offsets;
  xa.active = w.active;
  xa.n_active = w.n_active;
  xa.row_tok = w.row_tok;
  xa.row_w = w.row_w;
  xa.act = w.act;
  xa.rows_out = w.rows_out;
  xa.max_units = TK < E ? TK : E;
  xa.path = path;
  xa.distinct_ids = 1;  // the layer's own top-k picks distinct experts per token

  hipError_t e;
  const bool w8a8 = opts && opts->act_quant;
  if (w8a8) {
    xa.qx = w.qx;
    xa.dx = w.dx;
    xa.qa = w.qa;
    xa.da = w.da;
    if (!w8a8_ok(xa)) return MOE_ERR_UNSUPPORTED;
  }
  const bool decode_batch = T <= kFusedTokens && path != MOE_PATH_PREFILL && !w8a8;
  // prompt batches on the prefill GEMM pair or the W8A8 GEMMs keep the
  // expert rows in fp16 between the down projection and the combine
  xa.rows_f16 = !decode_batch && !mfma_decode_ok(xa) && (w8a8 || down_rows_f16_ok(xa)) ? 1 : 0;
  if (decode_batch) {
    // decode batch: the router's partial logits; the top-k and the
    // permutation then run inside the gate/up kernel when it is the
    // matrix-core one, else in one block of their own
    RouteFusedArgs fa{};
    fa.router_w = L->router_w;
    fa.router_bias = L->router_bias;
    fa.x = x_bf16;
    fa.T = T;
    fa.H = H;
    fa.E = E;
    fa.K = K;
    fa.renorm = L->renorm;
    fa.Hs = route_fused_slice(H);
    fa.S = H / fa.Hs;
    fa.logits = nullptr;
    fa.ids = ids;
    fa.w = tw;
    fa.part = w.part;
    fa.counts = w.counts;
    fa.offsets = w.offsets;
    fa.row_tok = w.row_tok;
    fa.inv_pos = w.inv_pos;
    fa.active = w.active;
    fa.n_active = w.n_active;
    fa.row_w = w.row_w;
    fa.units = w.units;
    fa.gate_w = L->shared_gate_w;
    fa.gate = w.gate;
    fa.Ep = router_rows(L);
    fa.tail_skip = opts ? opts->tail_skip : 0;
    xa.route_here = (mfma_decode_ok(xa) && E <= 256) ? 1 : 0;
    if (xa.route_here) xa.units = w.units;  // published by the gate/up kernel's routing
    if (xa.route_here && link.route_ready) {
      // the previous layer's combine wrote this call's whole router product
      // (one slice): the gate/up kernel's routing reads it as it is
      fa.S = 1;
      fa.Hs = H;
      fa.sorted = sorted_groups(L, w.part, T);
      xa.route = fa;
      e = hipSuccess;
    } else {
      xa.route = fa;
      StageMark m(ev, MOE_STAGE_ROUTE, s);
      e = xa.route_here ? launch_route_partial(fa, s) : launch_route_fused(fa, s);
    }
  } else {
    // (prompt batches: tail-skip leaves them untouched)
    // (the router GEMM's slices are added by the top-k kernel, which then
    // has no logits to write for the layer)
    float *lg = router_partial_floats(T, H, E, path) ? nullptr : w.logits;
    RouteArgs ra{L->router_w, L->router_bias, x_bf16, T, H, E, K, L->renorm, lg, ids, tw, w.x16, path,
                 L->shared_gate_w, w.gate, w.rpart};
    if (router_writes_x16(ra)) {
      xa.x16 = w.x16;
      xa.queue = w.control;
    }
    {
      StageMark m(ev, MOE_STAGE_ROUTE, s);
      e = launch_router_logits(ra, s);
      if (e == hipSuccess) e = launch_topk(ra, s);
    }
    if (e != hipSuccess) return MOE_ERR_HIP;
    PermuteArgs pa{};
    pa.ids = ids;
    pa.w = tw;
    pa.T = T;
    pa.K = K;
    pa.E = E;
    pa.counts = w.counts;
    pa.offsets = w.offsets;
    pa.row_tok = w.row_tok;
    pa.row_w = w.row_w;
    pa.inv_pos = w.inv_pos;
    pa.active = w.active;
    pa.n_active = w.n_active;
    pa.rank = w.rank;
    pa.tile_hist = w.tile_hist;
    StageMark m(ev, MOE_STAGE_PERMUTE, s);
    e = launch_permute(pa, s);
  }
  if (e != hipSuccess) return MOE_ERR_HIP;

  if (w8a8) {
    // the W8A8 expert products (gate/up and down record their stages' events)
    StageMark mg(ev, MOE_STAGE_GATEUP, s, true);
    StageMark md(ev, MOE_STAGE_DOWN, s, true);
    e = launch_w8a8(xa, s, ev.of(MOE_STAGE_GATEUP), ev.of(MOE_STAGE_DOWN));
  } else {
    StageMark m(ev, MOE_STAGE_GATEUP, s, true);
    xa.ev = ev.of(MOE_STAGE_GATEUP);
    e = launch_gateup(xa, s);
  }
  if (e != hipSuccess) return MOE_ERR_HIP;
  if (xa.route_here && (!res || !res->normed_out) && down_combine_ok(xa, K)) {
    // a few tokens: down projection and combine in one launch (the down
    // stage's events bracket it; the combine stage has no launch of its own)
    xa.ev = ev.of(MOE_STAGE_DOWN);
    DownCombineArgs d{xa, w.units, w.inv_pos, K, E, y, res ? res->residual_in : nullptr,
                      res ? res->residual_out : nullptr, L->shared_gate_w ? w.gate : nullptr};
    return hip_status(launch_down_combine(d, s));
  }
  if (!w8a8) {
    StageMark m(ev, MOE_STAGE_DOWN, s, true);
    xa.ev = ev.of(MOE_STAGE_DOWN);
    e = launch_down(xa, s);
  }
  if (e != hipSuccess) return MOE_ERR_HIP;

  // fp16 expert rows (prefill GEMM pair, W8A8): the shared expert's rows
  // follow the routed ones in the same element size
  const float *shared_rows =
      !has_shared ? nullptr
      : xa.rows_f16 ? reinterpret_cast<const float *>(reinterpret_cast<const uint16_t *>(w.rows_out) +
                                                      static_cast<size_t>(TK) * H)
                    : w.rows_out + static_cast<size_t>(TK) * H;
  CombineArgs ca = combine_args(w.rows_out, w.inv_pos, T, K, H, shared_rows, L->shared_gate_w ? w.gate : nullptr, y, res);
  ca.rows_f16 = xa.rows_f16;
  StageMark m(ev, MOE_STAGE_COMBINE, s);
  // (the combine's blocks of one token all read the residual and one writes
  // it, so the fused form needs distinct residual buffers)
  if (link.next && xa.route_here && !xa.rows_f16 && res && res->normed_out && res->residual_in != res->residual_out &&
      combine_route_ok(H)) {
    // the next layer's router product, from the normalised row this
    // combine forms, into the workspace's partial-logit area
    const moe_layer *N = link.next;
    CombineRouteArgs cr{ca, N->router_w, N->shared_gate_w, N->n_experts, router_rows(N), w.part, N->router_bias,
                        sorted_groups(N, w.part, T)};
    e = launch_combine_route(cr, s);
    if (e == hipSuccess && link.fused) *link.fused = true;
    return hip_status(e);
  }
  return hip_status(launch_combine(ca, s));
}

// Layers a stack call can chain: the shapes that decide the workspace carve
// and the decode kernels' choice are equal.
bool same_shape(const moe_layer *a, const moe_layer *b) {
  auto ex_eq = [](const moe_experts &p, const moe_experts &q) {
    return p.n_experts == q.n_experts && p.fmt == q.fmt && p.ffn == q.ffn;
  };
  return a->hidden == b->hidden && a->n_experts == b->n_experts && a->top_k == b->top_k && a->renorm == b->renorm &&
         ex_eq(a->routed, b->routed) && ex_eq(a->shared, b->shared) &&
         (a->shared_gate_w != nullptr) == (b->shared_gate_w != nullptr);
}

}  // namespace

int moe_layer_forward_ex(const moe_layer *L, const uint16_t *x_bf16, int32_t T, float *y, const moe_residual *res,
                         int32_t *topk_ids, float *topk_w, void *ws, size_t ws_bytes, const moe_forward_opts *opts,
                         void *stream) {
  return layer_forward(L, x_bf16, T, y, res, topk_ids, topk_w, ws, ws_bytes, opts, stream, StackLink{});
}

int moe_stack_forward(const moe_layer *layers, int32_t n_layers, const uint16_t *x_bf16, int32_t T,
                      const uint16_t *residual_in, uint16_t *residual_out, uint16_t *normed_out, float eps, float *y,
                      int32_t *topk_ids, float *topk_w, void *ws, size_t ws_bytes, void *stream) {
  if (!layers || n_layers <= 0 || T < 0) return MOE_ERR_INVALID_ARG;
  if (!residual_in || !residual_out || !normed_out || !(eps >= 0.f)) return MOE_ERR_INVALID_ARG;
  for (int32_t l = 0; l < n_layers; ++l) {
    const int rc = check_layer(&layers[l]);
    if (rc != MOE_OK) return rc;
    if (l > 0 && !same_shape(&layers[0], &layers[l])) return MOE_ERR_INVALID_ARG;
  }
  if (T == 0) return MOE_OK;
  // every call checks the workspace, the buffers and their alignment itself
  if (!ws || !aligned(ws, 256)) return MOE_ERR_WORKSPACE;
  const LayerWs w = carve_layer(&layers[0], T, ws);
  if (ws_bytes < w.bytes) return MOE_ERR_WORKSPACE;
  // residual buffers: layer l reads R_l and writes R_(l+1), R_0 = residual_in,
  // R_n = residual_out, and the others alternate between residual_out and
  // the workspace's copy so that a layer reads and writes different ones
  auto rbuf = [&](int32_t l) -> uint16_t * { return (n_layers - l) % 2 == 0 ? residual_out : w.rstack; };
  bool ready = false;
  for (int32_t l = 0; l < n_layers; ++l) {
    moe_residual res{l == 0 ? residual_in : rbuf(l), rbuf(l + 1), normed_out, eps, 0};
    const bool last = l + 1 == n_layers;
    bool fused = false;
    StackLink link;
    link.route_ready = ready;
    link.next = last ? nullptr : &layers[l + 1];
    link.fused = &fused;
    const int rc = layer_forward(&layers[l], l == 0 ? x_bf16 : normed_out, T, y, &res, last ? topk_ids : nullptr,
                                 last ? topk_w : nullptr, ws, ws_bytes, nullptr, stream, link);
    if (rc != MOE_OK) return rc;
    ready = fused;
  }
  return MOE_OK;
}

int moe_layer_forward(const moe_layer *L, const uint16_t *x_bf16, int32_t T, float *y, const moe_residual *res,
                      int32_t *topk_ids, float *topk_w, void *ws, size_t ws_bytes, void *stream) {
  return moe_layer_forward_ex(L, x_bf16, T, y, res, topk_ids, topk_w, ws, ws_bytes, nullptr, stream);
}

}  // extern "C"
