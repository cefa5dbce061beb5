// CPU oracle for the routed mixture-of-experts FFN layer.
//
// TEST INFRASTRUCTURE ONLY: plain, slow, double-precision code that states
// what the layer computes.  Only the tests, the smoke check and the
// benchmark's CPU-baseline leg may call it.  It shares no code with the GPU
// library.
//
// What it follows (page titles and sections of the source pages):
//  * "Qwen3.6-35B-A3B: pictures, several requests at once and speed",
//    introduction: a 256-expert, top-8 mixture of experts; Speed (0.1.45):
//    the shared expert's gate+up+SwiGLU run beside the routed experts and the
//    "MoE end" sums them.
//  * "qwen36: CUDA VRAM expert tier", How it works: the shared expert is
//    computed alongside the routed ones, and the placement of an expert's
//    weights leaves both the routing and the arithmetic unchanged (the result
//    is a pure function of the inputs, whatever the schedule).
//  * "Models and backends", What was tuned: ties among the largest values
//    go to the first (lowest-index) one; tail-skip section: the experts
//    computed keep the weights the router gave them.
//  * "Every Public GGUF of This Model Is Missing Its Head", section 5: raw
//    Q4 nibbles are offset-binary (one XOR with 0x8 per nibble gives the
//    signed value), i.e. stored as q + 8.
// Variants (oracle_opts, shared gate):
//  * "Qwen3.6-35B-A3B: pictures, several requests at once and speed",
//    Speed (0.1.45): the router and the shared expert's gate are one product
//    (a gate row beside the router rows); the gate scales the shared
//    expert's output through a sigmoid.
//  * "Models and backends", What was tuned, the tail-skip passage and its
//    table: an expert that every token of a call ranks at place N+1 or later
//    is left out, and the experts computed keep the router's weights.
//  * "Strata on an Intel Arc", Arc Pro B70: the fused int8 expert path for
//    the prompt; "Models and backends", How each backend was checked: the
//    engines quantise activations to 8 bits at every quantised matrix.  Here
//    one symmetric scale per row (a token's input, or one expert's SwiGLU
//    row), every quantiser decision in float32.
// The remaining steps (softmax router, renormalised top-k weights, SwiGLU
// experts, weighted combine plus an always-on shared expert, int8 per-row
// and int4 32-block scaling) are the plain definition of the layer.
#include "moe_oracle.h"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <thread>
#include <vector>

namespace {

// ---- IEEE bit layouts -------------------------------------------------------

// bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits.
double bf16_value(uint16_t b) {
  const int sign = b >> 15;
  const int ex = (b >> 7) & 0xFF;
  const int fr = b & 0x7F;
  double v;
  if (ex == 0)
    v = std::ldexp(static_cast<double>(fr), -126 - 7);  // 0.fraction * 2^-126
  else if (ex == 0xFF)
    v = fr ? std::nan("") : INFINITY;
  else
    v = std::ldexp(static_cast<double>(128 + fr), ex - 127 - 7);  // 1.fraction * 2^(ex-127)
  return sign ? -v : v;
}

// binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
double f16_value(uint16_t h) {
  const int sign = h >> 15;
  const int ex = (h >> 10) & 0x1F;
  const int fr = h & 0x3FF;
  double v;
  if (ex == 0)
    v = std::ldexp(static_cast<double>(fr), -14 - 10);
  else if (ex == 0x1F)
    v = fr ? std::nan("") : INFINITY;
  else
    v = std::ldexp(static_cast<double>(1024 + fr), ex - 15 - 10);
  return sign ? -v : v;
}

// Nearest bfloat16, ties to even.  The grid spacing at |v| in [2^e, 2^(e+1))
// is 2^(e-7); below 2^-126 it is the subnormal spacing 2^-133.
uint16_t bf16_round(double v) {
  if (std::isnan(v)) return 0x7FC0;
  const uint16_t sign = std::signbit(v) ? 0x8000 : 0;
  double a = std::fabs(v);
  if (a == 0.0) return sign;
  if (std::isinf(a)) return sign | 0x7F80;
  int e2;
  std::frexp(a, &e2);
  int e = e2 - 1;
  if (e < -126) e = -126;
  const double spacing = std::ldexp(1.0, e - 7);
  const double q = std::nearbyint(a / spacing);  // current mode: nearest, ties to even
  const double r = q * spacing;                  // exactly a bfloat16 value (or overflow)
  const double max_bf16 = std::ldexp(255.0, 127 - 7);
  if (r > max_bf16) return sign | 0x7F80;
  if (r < std::ldexp(1.0, -126)) return sign | static_cast<uint16_t>(q);  // subnormal fraction
  std::frexp(r, &e2);
  e = e2 - 1;
  const int frac = static_cast<int>(std::ldexp(r, 7 - e)) - 128;
  return sign | static_cast<uint16_t>((e + 127) << 7) | static_cast<uint16_t>(frac);
}

// ---- weight formats -----------------------------------------------------------

// W[n][k] of matrix e, exactly, or NaN for a forbidden nibble.
double weight_at(int32_t fmt, const void *q, const void *s, int64_t e, int64_t rows, int64_t kin, int64_t n,
                 int64_t k) {
  if (fmt == 1) {
    const int8_t *qq = static_cast<const int8_t *>(q);
    const float *ss = static_cast<const float *>(s);
    return static_cast<double>(qq[(e * rows + n) * kin + k]) * static_cast<double>(ss[e * rows + n]);
  }
  if (fmt == 2) {
    const uint8_t *qq = static_cast<const uint8_t *>(q);
    const uint16_t *ss = static_cast<const uint16_t *>(s);
    const uint8_t byte = qq[(e * rows + n) * (kin / 2) + k / 2];
    const int nib = (k % 2 == 1) ? (byte >> 4) : (byte & 0xF);
    if (nib == 0) return std::nan("");
    const int qv = nib - 8;
    return static_cast<double>(qv) * f16_value(ss[(e * rows + n) * (kin / 32) + k / 32]);
  }
  return std::nan("");
}

double silu(double g) { return g / (1.0 + std::exp(-g)); }

double sigmoid(double z) { return 1.0 / (1.0 + std::exp(-z)); }

// Symmetric int8 quantisation of one row in float32 (see the header).
void quantize_row(const float *v, int64_t n, int8_t *q, float *d) {
  float amax = 0.0f;
  for (int64_t i = 0; i < n; ++i) amax = std::max(amax, std::fabs(v[i]));
  if (amax == 0.0f) {
    for (int64_t i = 0; i < n; ++i) q[i] = 0;
    *d = 0.0f;
    return;
  }
  const float inv = 127.0f / amax;
  *d = amax / 127.0f;
  for (int64_t i = 0; i < n; ++i) {
    const float p = v[i] * inv;  // one float32 rounding
    float r = std::nearbyint(p);  // ties to even (the default rounding mode)
    r = std::min(127.0f, std::max(-127.0f, r));
    q[i] = static_cast<int8_t>(r);
  }
}

// A row after quantisation and back: q * d, exactly, in double.
void quantize_dequantize(const float *v, int64_t n, double *out) {
  std::vector<int8_t> q(n);
  float d = 0.0f;
  quantize_row(v, n, q.data(), &d);
  for (int64_t i = 0; i < n; ++i) out[i] = static_cast<double>(q[i]) * static_cast<double>(d);
}

// out = D (silu(G x) * (U x)) for expert e.  With quant_a the SwiGLU row
// is rounded to float32 (the precision the GPU holds it in) and quantised
// per row before the down projection.  Returns false on a NaN weight.
bool expert_apply(const oracle_experts &W, int32_t e, const double *x, double *out, bool quant_a = false) {
  const int64_t H = W.hidden, F = W.ffn;
  std::vector<double> a(F);
  bool ok = true;
  for (int64_t f = 0; f < F; ++f) {
    double g = 0.0, u = 0.0;
    for (int64_t h = 0; h < H; ++h) {
      const double wg = weight_at(W.fmt, W.gate_q, W.gate_s, e, F, H, f, h);
      const double wu = weight_at(W.fmt, W.up_q, W.up_s, e, F, H, f, h);
      g += wg * x[h];
      u += wu * x[h];
    }
    if (std::isnan(g) || std::isnan(u)) ok = false;
    a[f] = silu(g) * u;
  }
  if (quant_a) {
    std::vector<float> a32(F);
    for (int64_t f = 0; f < F; ++f) a32[f] = static_cast<float>(a[f]);
    quantize_dequantize(a32.data(), F, a.data());
  }
  for (int64_t h = 0; h < H; ++h) {
    double o = 0.0;
    for (int64_t f = 0; f < F; ++f) o += weight_at(W.fmt, W.down_q, W.down_s, e, H, F, h, f) * a[f];
    out[h] = o;
  }
  return ok;
}

void token_logits(const oracle_layer &L, const double *x, double *l) {
  for (int e = 0; e < L.n_experts; ++e) {
    double acc = 0.0;
    for (int h = 0; h < L.hidden; ++h)
      acc += static_cast<double>(L.router_w[static_cast<int64_t>(e) * L.hidden + h]) * x[h];
    if (L.router_bias) acc += static_cast<double>(L.router_bias[e]);
    l[e] = acc;
  }
}

// Order experts by (logit descending, index ascending) and keep the first K.
void token_select(const double *l, int32_t E, int32_t K, int32_t renorm, int32_t *ids, double *w) {
  std::vector<int32_t> order(E);
  for (int32_t e = 0; e < E; ++e) order[e] = e;
  std::sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
    if (l[a] != l[b]) return l[a] > l[b];
    return a < b;
  });
  for (int32_t k = 0; k < K; ++k) ids[k] = order[k];
  // Softmax over all E then renormalised over the chosen K equals a softmax
  // over the K chosen logits; without renormalisation the denominator runs
  // over every expert.  The largest logit is subtracted for range only.
  const double m = l[order[0]];
  double denom = 0.0;
  if (renorm) {
    for (int32_t k = 0; k < K; ++k) denom += std::exp(l[ids[k]] - m);
  } else {
    for (int32_t e = 0; e < E; ++e) denom += std::exp(l[e] - m);
  }
  for (int32_t k = 0; k < K; ++k) w[k] = std::exp(l[ids[k]] - m) / denom;
}

template <typename Fn>
void parallel_over(int32_t n, int32_t nthreads, Fn fn) {
  if (nthreads <= 0) nthreads = static_cast<int32_t>(std::max(1u, std::thread::hardware_concurrency()));
  nthreads = std::min(nthreads, std::max(n, 1));
  if (nthreads <= 1) {
    for (int32_t i = 0; i < n; ++i) fn(i);
    return;
  }
  std::vector<std::thread> pool;
  for (int32_t t = 0; t < nthreads; ++t)
    pool.emplace_back([=, &fn] {
      for (int32_t i = t; i < n; i += nthreads) fn(i);
    });
  for (auto &th : pool) th.join();
}

}  // namespace

extern "C" {

double oracle_bf16_to_double(uint16_t bits) { return bf16_value(bits); }
double oracle_f16_to_double(uint16_t bits) { return f16_value(bits); }
uint16_t oracle_double_to_bf16(double v) { return bf16_round(v); }
int32_t oracle_threads(void) {
  return static_cast<int32_t>(std::max(1u, std::thread::hardware_concurrency()));
}

double oracle_weight(int32_t fmt, const void *q, const void *s, int64_t e, int64_t rows, int64_t kin, int64_t n,
                     int64_t k) {
  return weight_at(fmt, q, s, e, rows, kin, n, k);
}

int oracle_dequant(int32_t fmt, const void *q, const void *s, int64_t n_mat, int64_t rows, int64_t kin,
                   double *out) {
  int rc = 0;
  for (int64_t e = 0; e < n_mat; ++e)
    for (int64_t n = 0; n < rows; ++n)
      for (int64_t k = 0; k < kin; ++k) {
        const double v = weight_at(fmt, q, s, e, rows, kin, n, k);
        if (std::isnan(v)) rc = -1;
        out[(e * rows + n) * kin + k] = v;
      }
  return rc;
}

void oracle_router_logits(const oracle_layer *L, const uint16_t *x_bf16, int32_t T, double *logits) {
  std::vector<double> x(L->hidden);
  for (int32_t t = 0; t < T; ++t) {
    for (int h = 0; h < L->hidden; ++h) x[h] = bf16_value(x_bf16[static_cast<int64_t>(t) * L->hidden + h]);
    token_logits(*L, x.data(), logits + static_cast<int64_t>(t) * L->n_experts);
  }
}

void oracle_select(const double *logits, int32_t T, int32_t E, int32_t K, int32_t renorm, int32_t *ids,
                   double *w) {
  for (int32_t t = 0; t < T; ++t)
    token_select(logits + static_cast<int64_t>(t) * E, E, K, renorm, ids + static_cast<int64_t>(t) * K,
                 w + static_cast<int64_t>(t) * K);
}

int oracle_expert_apply(const oracle_experts *W, int32_t e, const double *x, double *out) {
  return expert_apply(*W, e, x, out) ? 0 : -1;
}

void oracle_permute(const int32_t *ids, const float *w, int32_t T, int32_t K, int32_t E, int32_t *counts,
                    int32_t *offsets, int32_t *row_tok, float *row_w, int32_t *inv_pos, int32_t *active,
                    int32_t *n_active) {
  for (int32_t e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t p = 0; p < static_cast<int64_t>(T) * K; ++p) counts[ids[p]] += 1;
  offsets[0] = 0;
  for (int32_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int32_t na = 0;
  for (int32_t e = 0; e < E; ++e) {
    if (counts[e] > 0) active[na++] = e;
    int32_t r = offsets[e];
    for (int32_t t = 0; t < T; ++t)
      for (int32_t k = 0; k < K; ++k) {
        const int64_t p = static_cast<int64_t>(t) * K + k;
        if (ids[p] != e) continue;
        row_tok[r] = t;
        if (row_w) row_w[r] = w ? w[p] : 1.0f;
        inv_pos[p] = r;
        ++r;
      }
  }
  *n_active = na;
}

int oracle_layer_forward_ex(const oracle_layer *L, const uint16_t *x_bf16, int32_t T, const int32_t *ids_in,
                            const oracle_opts *opts, double *y, int32_t *ids_out, double *w_out, double *logits_out,
                            int32_t nthreads) {
  const int32_t H = L->hidden, E = L->n_experts, K = L->top_k;
  const int32_t tail_skip = opts ? opts->tail_skip : 0;
  const bool act_quant = opts && opts->act_quant;
  // Routing of every token first: the tail-skip rule looks at the whole call.
  std::vector<int32_t> ids(static_cast<size_t>(T) * K);
  std::vector<double> w(static_cast<size_t>(T) * K), gate(T, 1.0);
  parallel_over(T, nthreads, [&](int32_t t) {
    std::vector<double> x(H), l(E);
    int32_t *id = ids.data() + static_cast<int64_t>(t) * K;
    double *wt = w.data() + static_cast<int64_t>(t) * K;
    for (int h = 0; h < H; ++h) x[h] = bf16_value(x_bf16[static_cast<int64_t>(t) * H + h]);
    token_logits(*L, x.data(), l.data());
    token_select(l.data(), E, K, L->renorm, id, wt);
    if (ids_in) {
      // Selection supplied by the caller (a near-tie token may legitimately
      // pick either expert): weights from the logits at the given ids.
      const int32_t *sel = ids_in + static_cast<int64_t>(t) * K;
      double m = l[sel[0]];
      for (int32_t k = 1; k < K; ++k) m = std::max(m, l[sel[k]]);
      double denom = 0.0;
      if (L->renorm)
        for (int32_t k = 0; k < K; ++k) denom += std::exp(l[sel[k]] - m);
      else
        for (int32_t e = 0; e < E; ++e) denom += std::exp(l[e] - m);
      for (int32_t k = 0; k < K; ++k) {
        id[k] = sel[k];
        wt[k] = std::exp(l[sel[k]] - m) / denom;
      }
    }
    if (L->shared && L->shared_gate_w) {
      // the shared expert's gate: one more row of the router's product
      double z = 0.0;
      for (int h = 0; h < H; ++h) z += static_cast<double>(L->shared_gate_w[h]) * x[h];
      gate[t] = sigmoid(z);
    }
    if (logits_out)
      for (int32_t e = 0; e < E; ++e) logits_out[static_cast<int64_t>(t) * E + e] = l[e];
  });
  // Tail-skip: an expert is kept when some token of the call ranks it among
  // its first tail_skip picks.
  std::vector<char> keep(E, 1);
  if (tail_skip > 0) {
    std::fill(keep.begin(), keep.end(), 0);
    for (int32_t t = 0; t < T; ++t)
      for (int32_t k = 0; k < std::min(tail_skip, K); ++k) keep[ids[static_cast<int64_t>(t) * K + k]] = 1;
  }
  std::vector<int> bad(T, 0);
  parallel_over(T, nthreads, [&](int32_t t) {
    std::vector<double> x(H), o(H), acc(H, 0.0);
    for (int h = 0; h < H; ++h) x[h] = bf16_value(x_bf16[static_cast<int64_t>(t) * H + h]);
    if (act_quant) {
      // the token's input to every expert, quantised once per row
      std::vector<float> x32(H);
      for (int h = 0; h < H; ++h) x32[h] = static_cast<float>(x[h]);  // exact: x is bf16
      quantize_dequantize(x32.data(), H, x.data());
    }
    for (int32_t k = 0; k < K; ++k) {
      const int32_t e = ids[static_cast<int64_t>(t) * K + k];
      if (!keep[e]) continue;
      if (!expert_apply(L->routed, e, x.data(), o.data(), act_quant)) bad[t] = 1;
      const double wk = w[static_cast<int64_t>(t) * K + k];
      for (int h = 0; h < H; ++h) acc[h] += wk * o[h];
    }
    if (L->shared) {
      if (!expert_apply(*L->shared, 0, x.data(), o.data(), act_quant)) bad[t] = 1;
      if (L->shared_gate_w) {
        for (int h = 0; h < H; ++h) acc[h] += gate[t] * o[h];
      } else {
        for (int h = 0; h < H; ++h) acc[h] += o[h];
      }
    }
    for (int h = 0; h < H; ++h) y[static_cast<int64_t>(t) * H + h] = acc[h];
    for (int32_t k = 0; k < K; ++k) {
      if (ids_out) ids_out[static_cast<int64_t>(t) * K + k] = ids[static_cast<int64_t>(t) * K + k];
      if (w_out) w_out[static_cast<int64_t>(t) * K + k] = w[static_cast<int64_t>(t) * K + k];
    }
  });
  for (int32_t t = 0; t < T; ++t)
    if (bad[t]) return -1;
  return 0;
}

int oracle_layer_forward(const oracle_layer *L, const uint16_t *x_bf16, int32_t T, const int32_t *ids_in,
                         double *y, int32_t *ids_out, double *w_out, double *logits_out, int32_t nthreads) {
  return oracle_layer_forward_ex(L, x_bf16, T, ids_in, nullptr, y, ids_out, w_out, logits_out, nthreads);
}

void oracle_quantize_row(const float *v, int64_t n, int8_t *q, float *d) { quantize_row(v, n, q, d); }

int oracle_expert_rows(const oracle_experts *W, const uint16_t *x_bf16, const int32_t *offsets,
                       const int32_t *row_tok, const float *row_w, int32_t n_rows, double *rows_out,
                       int32_t nthreads) {
  const int32_t H = W->hidden;
  std::vector<int> bad(n_rows, 0);
  parallel_over(n_rows, nthreads, [&](int32_t r) {
    int32_t e = 0;
    while (e < W->n_experts && !(offsets[e] <= r && r < offsets[e + 1])) ++e;
    if (e == W->n_experts) {
      bad[r] = 1;
      return;
    }
    const int32_t t = row_tok ? row_tok[r] : r;
    std::vector<double> x(H), o(H);
    for (int h = 0; h < H; ++h) x[h] = bf16_value(x_bf16[static_cast<int64_t>(t) * H + h]);
    if (!expert_apply(*W, e, x.data(), o.data())) bad[r] = 1;
    const double wr = row_w ? static_cast<double>(row_w[r]) : 1.0;
    for (int h = 0; h < H; ++h) rows_out[static_cast<int64_t>(r) * H + h] = wr * o[h];
  });
  for (int32_t r = 0; r < n_rows; ++r)
    if (bad[r]) return -1;
  return 0;
}

void oracle_residual(const uint16_t *x_bf16, const double *y, int64_t n, uint16_t *x_next) {
  for (int64_t i = 0; i < n; ++i) x_next[i] = bf16_round(bf16_value(x_bf16[i]) + y[i]);
}

// RMS normalisation of a layer stack's residual (no learned gain): the
// pages' model normalises each layer's input ("Qwen3.6-35B-A3B: pictures,
// several requests at once and speed", Speed (0.1.45)).
void oracle_rmsnorm(const uint16_t *r_bf16, int64_t T, int64_t H, double eps, uint16_t *out) {
  for (int64_t t = 0; t < T; ++t) {
    double ss = 0.0;
    for (int64_t h = 0; h < H; ++h) {
      const double v = bf16_value(r_bf16[t * H + h]);
      ss += v * v;
    }
    const double scale = 1.0 / std::sqrt(ss / static_cast<double>(H) + eps);
    for (int64_t h = 0; h < H; ++h) out[t * H + h] = bf16_round(bf16_value(r_bf16[t * H + h]) * scale);
  }
}

}  // extern "C"
