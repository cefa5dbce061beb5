/*
 * CPU oracle for the routed mixture-of-experts FFN layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Plain, slow, double-precision code that states
 * what the layer computes.  It shares no code with the GPU library and is
 * called only by the tests, the smoke check and the benchmark's CPU-baseline
 * leg.  No product path may link or call it.
 *
 * All pointers are host memory, row-major, the reduction dimension
 * contiguous.  Weight formats:
 *   fmt 1 (int8, per-row scale): q int8 [E][N][Kin], s float32 [E][N];
 *          W[n][k] = q[n][k] * s[n].
 *   fmt 2 (int4, 32-element blocks): q uint8 [E][N][Kin/2], s binary16 bits
 *          [E][N][Kin/32]; byte j holds element 2j in its low nibble and
 *          2j+1 in its high nibble, stored as q + 8 (q in [-7, 7]);
 *          W[n][k] = q[n][k] * s[n][k/32].
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int32_t fmt;       /* 1 = int8 per-row, 2 = int4 block-32 */
  int32_t n_experts; /* experts held by the arrays */
  int32_t hidden;    /* H */
  int32_t ffn;       /* F */
  const void *gate_q, *gate_s; /* [E][F][H] */
  const void *up_q, *up_s;     /* [E][F][H] */
  const void *down_q, *down_s; /* [E][H][F] */
} oracle_experts;

typedef struct {
  int32_t hidden, n_experts, top_k, renorm; /* renorm 1: weights = softmax over the K chosen */
  const float *router_w;    /* float32 [E][H] */
  const float *router_bias; /* float32 [E] or NULL */
  oracle_experts routed;
  const oracle_experts *shared; /* NULL: no shared expert */
  /* float32 [H] or NULL: the shared expert's gate row; its output is then
   * scaled by sigmoid(sum_h g[h] x[h]) instead of 1 */
  const float *shared_gate_w;
} oracle_layer;

/* Variants of a layer call (all zero = the plain layer). */
typedef struct {
  /* 0: off.  N > 0: an expert that no token of the call ranks among its
   * first N picks is not computed; the others keep their router weights
   * (no renormalisation). */
  int32_t tail_skip;
  /* 0: bf16 activations as given.  1: the input of every expert's gate/up
   * and of its down projection is first quantised per row to int8 with
   * oracle_quantize_row (the W8A8 variant). */
  int32_t act_quant;
} oracle_opts;

/* IEEE decoders written from the bit layouts. */
double oracle_bf16_to_double(uint16_t bits);
double oracle_f16_to_double(uint16_t bits);
/* Round a double to the nearest bfloat16 (ties to even). */
uint16_t oracle_double_to_bf16(double v);

/* Element (n, k) of expert e's matrix in format fmt, exactly in double.
 * Returns NaN for an int4 nibble of 0 (q = -8 is outside the format). */
double oracle_weight(int32_t fmt, const void *q, const void *s, int64_t e, int64_t rows, int64_t kin,
                     int64_t n, int64_t k);
/* Dense dequantisation of a whole [E][N][Kin] tensor (0 on success, -1 on a
 * nibble of 0). */
int oracle_dequant(int32_t fmt, const void *q, const void *s, int64_t n_mat, int64_t rows, int64_t kin,
                   double *out);

/* logits[t][e] = sum_h Wr[e][h] * x[t][h] (+ bias[e]) */
void oracle_router_logits(const oracle_layer *L, const uint16_t *x_bf16, int32_t T, double *logits);
/* Top-K by a full sort of (logit desc, index asc); weights per renorm. */
void oracle_select(const double *logits, int32_t T, int32_t E, int32_t K, int32_t renorm, int32_t *ids,
                   double *w);
/* One expert on one token: out[h] = (D (silu(G x) * (U x)))[h]. */
int oracle_expert_apply(const oracle_experts *W, int32_t e, const double *x, double *out);
/* Token-by-expert permutation: counts[E], offsets[E+1], rows ordered by
 * expert then (t, k); row_tok[TK], row_w[TK] (w may be NULL), inv_pos[TK],
 * active[E] = experts with rows in increasing order, *n_active. */
void oracle_permute(const int32_t *ids, const float *w, int32_t T, int32_t K, int32_t E, int32_t *counts,
                    int32_t *offsets, int32_t *row_tok, float *row_w, int32_t *inv_pos, int32_t *active,
                    int32_t *n_active);
/* Whole layer: y[t] = sum_k w_k o_{ids_k}(x_t) + o_shared(x_t).  If
 * ids_in is non-NULL it overrides the selection (weights still come from
 * the router's logits at those ids).  ids_out/w_out/logits_out may be NULL.
 * nthreads <= 0 uses the machine's hardware concurrency.  Returns 0, or -1
 * on malformed weights. */
int oracle_layer_forward(const oracle_layer *L, const uint16_t *x_bf16, int32_t T, const int32_t *ids_in,
                         double *y, int32_t *ids_out, double *w_out, double *logits_out, int32_t nthreads);
/* oracle_layer_forward with the variants of `opts` (NULL = none). */
int oracle_layer_forward_ex(const oracle_layer *L, const uint16_t *x_bf16, int32_t T, const int32_t *ids_in,
                            const oracle_opts *opts, double *y, int32_t *ids_out, double *w_out, double *logits_out,
                            int32_t nthreads);
/* Per-row symmetric int8 quantisation, every step in float32 (the
 * precision the GPU takes the same decisions in): amax = max |v|; amax = 0
 * gives q = 0, d = 0; else inv = 127 / amax, d = amax / 127 (each one
 * correctly rounded division) and q[i] = round-half-even(v[i] * inv) (one
 * rounded product), clamped to [-127, 127].  The row is then q * d. */
void oracle_quantize_row(const float *v, int64_t n, int8_t *q, float *d);
/* rows_out[r] = row_w[r] * o_e(x_{row_tok[r]}) for the expert e whose
 * offsets range holds r (row_w NULL: weight 1; row_tok NULL: r). */
int oracle_expert_rows(const oracle_experts *W, const uint16_t *x_bf16, const int32_t *offsets,
                       const int32_t *row_tok, const float *row_w, int32_t n_rows, double *rows_out,
                       int32_t nthreads);
/* x_next = bf16_rne(x + y) elementwise. */
void oracle_residual(const uint16_t *x_bf16, const double *y, int64_t n, uint16_t *x_next);
/* out[t] = bf16(r[t] / sqrt(mean_h r[t][h]^2 + eps)) per row of H values. */
void oracle_rmsnorm(const uint16_t *r_bf16, int64_t T, int64_t H, double eps, uint16_t *out);
int32_t oracle_threads(void);

#ifdef __cplusplus
}
#endif
#endif
