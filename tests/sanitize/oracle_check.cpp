// Runs every entry point of the CPU oracle on small layers (int8 and int4
// weights, a shared expert with its gate row, a router bias, every variant)
// so that a build with AddressSanitizer and UndefinedBehaviorSanitizer sees
// each code path once.  Prints "ok" and exits 0 when every output is finite.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "moe_oracle.h"

namespace {

uint64_t g_state = 0x9E3779B97F4A7C15ull;
uint32_t next_u32() {  // xorshift64*, test data only
  g_state ^= g_state >> 12;
  g_state ^= g_state << 25;
  g_state ^= g_state >> 27;
  return static_cast<uint32_t>((g_state * 0x2545F4914F6CDD1Dull) >> 32);
}
float uniform(float lo, float hi) { return lo + (hi - lo) * (next_u32() >> 8) * (1.0f / 16777216.0f); }
uint16_t bf16_of(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return static_cast<uint16_t>((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}
uint16_t f16_of_small(float f) {  // positive normal values in [2^-14, 2)
  int e;
  const float m = std::frexp(f, &e);  // f = m 2^e, m in [0.5, 1)
  const uint32_t mant = static_cast<uint32_t>((m * 2.0f - 1.0f) * 1024.0f);
  return static_cast<uint16_t>(((e - 1 + 15) << 10) | (mant & 0x3FFu));
}

struct Experts {
  std::vector<int8_t> q8[3];
  std::vector<uint8_t> q4[3];
  std::vector<float> s8[3];
  std::vector<uint16_t> s4[3];
  oracle_experts o{};
};

// gate, up [E][F][H]; down [E][H][F]
void make_experts(Experts &x, int fmt, int E, int H, int F) {
  const int rows[3] = {F, F, H}, kin[3] = {H, H, F};
  x.o.fmt = fmt;
  x.o.n_experts = E;
  x.o.hidden = H;
  x.o.ffn = F;
  const void **qp[3] = {&x.o.gate_q, &x.o.up_q, &x.o.down_q};
  const void **sp[3] = {&x.o.gate_s, &x.o.up_s, &x.o.down_s};
  for (int m = 0; m < 3; ++m) {
    const size_t n = static_cast<size_t>(E) * rows[m] * kin[m];
    if (fmt == 1) {
      x.q8[m].resize(n);
      for (auto &v : x.q8[m]) v = static_cast<int8_t>(static_cast<int>(next_u32() % 255) - 127);
      x.s8[m].resize(static_cast<size_t>(E) * rows[m]);
      for (auto &v : x.s8[m]) v = uniform(0.5f, 1.5f) / (127.0f * std::sqrt(static_cast<float>(kin[m])));
      *qp[m] = x.q8[m].data();
      *sp[m] = x.s8[m].data();
    } else {
      x.q4[m].resize(n / 2);
      for (auto &v : x.q4[m]) v = static_cast<uint8_t>((1 + next_u32() % 15) | ((1 + next_u32() % 15) << 4));
      x.s4[m].resize(static_cast<size_t>(E) * rows[m] * (kin[m] / 32));
      for (auto &v : x.s4[m]) v = f16_of_small(uniform(0.5f, 1.5f) / (7.0f * std::sqrt(static_cast<float>(kin[m]))));
      *qp[m] = x.q4[m].data();
      *sp[m] = x.s4[m].data();
    }
  }
}

bool finite_all(const std::vector<double> &v) {
  for (double d : v)
    if (!std::isfinite(d)) return false;
  return true;
}

int run(int fmt) {
  const int H = 64, F = 32, E = 6, K = 2, T = 5;
  Experts routed, shared;
  make_experts(routed, fmt, E, H, F);
  make_experts(shared, fmt, 1, H, F);
  std::vector<float> rw(static_cast<size_t>(E) * H), bias(E), gate(H);
  for (auto &v : rw) v = uniform(-0.1f, 0.1f);
  for (auto &v : bias) v = uniform(-0.5f, 0.5f);
  for (auto &v : gate) v = uniform(-0.1f, 0.1f);
  oracle_layer L{};
  L.hidden = H;
  L.n_experts = E;
  L.top_k = K;
  L.renorm = 1;
  L.router_w = rw.data();
  L.router_bias = bias.data();
  L.routed = routed.o;
  L.shared = &shared.o;
  L.shared_gate_w = gate.data();
  std::vector<uint16_t> x(static_cast<size_t>(T) * H);
  for (auto &v : x) v = bf16_of(uniform(-2.0f, 2.0f));

  std::vector<double> y(static_cast<size_t>(T) * H), w(static_cast<size_t>(T) * K), lg(static_cast<size_t>(T) * E);
  std::vector<int32_t> ids(static_cast<size_t>(T) * K);
  for (int variant = 0; variant < 4; ++variant) {
    oracle_opts o{};
    o.tail_skip = variant == 1 ? 1 : 0;
    o.act_quant = variant == 2 ? 1 : 0;
    const int nthreads = variant == 3 ? 3 : 1;
    if (oracle_layer_forward_ex(&L, x.data(), T, nullptr, &o, y.data(), ids.data(), w.data(), lg.data(), nthreads))
      return 1;
    if (!finite_all(y) || !finite_all(w) || !finite_all(lg)) return 2;
  }
  if (oracle_layer_forward(&L, x.data(), T, ids.data(), y.data(), nullptr, nullptr, nullptr, 2)) return 3;

  std::vector<int32_t> counts(E), offsets(E + 1), row_tok(T * K), inv(T * K), active(E), n_active(1);
  std::vector<float> wf(T * K, 0.5f), row_w(T * K);
  oracle_permute(ids.data(), wf.data(), T, K, E, counts.data(), offsets.data(), row_tok.data(), row_w.data(),
                 inv.data(), active.data(), n_active.data());
  std::vector<double> rows(static_cast<size_t>(T) * K * H);
  if (oracle_expert_rows(&routed.o, x.data(), offsets.data(), row_tok.data(), row_w.data(), T * K, rows.data(), 2))
    return 4;
  if (!finite_all(rows)) return 5;

  std::vector<double> dq(static_cast<size_t>(E) * F * H);
  if (oracle_dequant(fmt, routed.o.gate_q, routed.o.gate_s, E, F, H, dq.data())) return 6;
  std::vector<uint16_t> xn(x.size()), rn(x.size());
  oracle_residual(x.data(), y.data(), static_cast<int64_t>(x.size()), xn.data());
  oracle_rmsnorm(xn.data(), T, H, 1e-6, rn.data());
  std::vector<float> v(33);
  for (auto &f : v) f = uniform(-3.0f, 3.0f);
  std::vector<int8_t> q(33);
  float d = 0.f;
  oracle_quantize_row(v.data(), 33, q.data(), &d);
  std::vector<float> zeros(7, 0.f);
  oracle_quantize_row(zeros.data(), 7, q.data(), &d);
  for (int b = 0; b < 65536; b += 97) {
    (void)oracle_bf16_to_double(static_cast<uint16_t>(b));
    (void)oracle_f16_to_double(static_cast<uint16_t>(b));
  }
  (void)oracle_double_to_bf16(3.25);
  return 0;
}

}  // namespace

int main() {
  for (int fmt = 1; fmt <= 2; ++fmt) {
    const int rc = run(fmt);
    if (rc) {
      std::printf("failed: fmt %d, step %d\n", fmt, rc);
      return rc;
    }
  }
  std::printf("ok\n");
  return 0;
}
