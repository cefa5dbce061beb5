// Drives the host side of the C ABI (argument validation, workspace sizing,
// status text) through every early-return path that needs no GPU, for a
// build of the library whose host code carries AddressSanitizer.  No call
// here launches work: each either returns an error or, with T = 0, returns
// before touching a device.  Prints "ok" and exits 0 when every status is
// the expected one.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <limits>

#include "moe.h"

namespace {

int g_fail = 0;
void expect(int got, int want, const char *what) {
  if (got != want) {
    std::printf("%s: got %d, want %d\n", what, got, want);
    ++g_fail;
  }
}

moe_layer fake_layer(int32_t H, int32_t E, int32_t K, int32_t F, int32_t fmt, bool shared) {
  const void *p = reinterpret_cast<const void *>(uintptr_t{1} << 20);  // aligned, never dereferenced
  moe_layer L;
  std::memset(&L, 0, sizeof(L));
  L.hidden = H;
  L.n_experts = E;
  L.top_k = K;
  L.renorm = 1;
  L.router_w = static_cast<const float *>(p);
  L.routed = moe_experts{fmt, E, F, 0, p, p, p, p, p, p};
  if (shared) L.shared = moe_experts{fmt, 1, F, 0, p, p, p, p, p, p};
  return L;
}

}  // namespace

int main() {
  void *p = reinterpret_cast<void *>(uintptr_t{1} << 20);
  for (int s = -8; s <= 2; ++s)
    expect(moe_status_string(s) && std::strlen(moe_status_string(s)) > 0, 1, "status text");

  // workspace sizes over many shapes, and zero for invalid layers
  for (int fmt = 1; fmt <= 2; ++fmt)
    for (int32_t T : {1, 2, 7, 16, 17, 64, 300, 2048, 8192}) {
      moe_layer L = fake_layer(2048, 256, 8, 512, fmt, true);
      expect(moe_workspace_bytes(&L, T) > 0, 1, "workspace bytes");
      expect(moe_route_workspace_bytes(&L, T) > 0, 1, "route workspace bytes");
      L = fake_layer(1024, 64, 4, fmt == 1 ? 256 : 512, fmt, false);  // int4 takes F % 512 == 0
      expect(moe_workspace_bytes(&L, T) > 0, 1, "workspace bytes, small layer");
    }
  {
    moe_layer L = fake_layer(2048, 256, 8, 512, 2, true);
    L.top_k = 0;
    expect(moe_workspace_bytes(&L, 4) == 0, 1, "K = 0");
    L = fake_layer(1000, 256, 8, 512, 2, true);
    expect(moe_workspace_bytes(&L, 4) == 0, 1, "H = 1000");
    L = fake_layer(2048, 256, 8, 512, 9, true);
    expect(moe_workspace_bytes(&L, 4) == 0, 1, "format 9");
    expect(moe_workspace_bytes(nullptr, 4) == 0, 1, "null layer");
  }
  expect(moe_permute_workspace_bytes(2048, 8, 256) > 0, 1, "permute workspace");
  expect(moe_expert_ffn_workspace_bytes(100, 512) > 0, 1, "expert workspace");

  // the layer: every rejection before a launch
  moe_layer L = fake_layer(2048, 256, 8, 512, 2, true);
  expect(moe_layer_forward(nullptr, static_cast<uint16_t *>(p), 4, static_cast<float *>(p), nullptr, nullptr,
                           nullptr, p, size_t{1} << 30, nullptr),
         MOE_ERR_INVALID_ARG, "null layer");
  expect(moe_layer_forward(&L, static_cast<uint16_t *>(p), 0, static_cast<float *>(p), nullptr, nullptr, nullptr,
                           nullptr, 0, nullptr),
         MOE_OK, "T = 0");
  expect(moe_layer_forward(&L, static_cast<uint16_t *>(p), -1, static_cast<float *>(p), nullptr, nullptr, nullptr,
                           p, size_t{1} << 30, nullptr),
         MOE_ERR_INVALID_ARG, "T < 0");
  expect(moe_layer_forward(&L, nullptr, 4, static_cast<float *>(p), nullptr, nullptr, nullptr, p, size_t{1} << 30,
                           nullptr),
         MOE_ERR_INVALID_ARG, "null x");
  expect(moe_layer_forward(&L, static_cast<uint16_t *>(p), 4, static_cast<float *>(p), nullptr, nullptr, nullptr,
                           p, 16, nullptr),
         MOE_ERR_WORKSPACE, "small workspace");
  moe_forward_opts o;
  std::memset(&o, 0, sizeof(o));
  o.path = 7;
  expect(moe_layer_forward_ex(&L, static_cast<uint16_t *>(p), 4, static_cast<float *>(p), nullptr, nullptr, nullptr,
                              p, size_t{1} << 30, &o, nullptr),
         MOE_ERR_INVALID_ARG, "bad path");
  std::memset(&o, 0, sizeof(o));
  o.tail_skip = -3;
  expect(moe_layer_forward_ex(&L, static_cast<uint16_t *>(p), 4, static_cast<float *>(p), nullptr, nullptr, nullptr,
                              p, size_t{1} << 30, &o, nullptr),
         MOE_ERR_INVALID_ARG, "bad tail-skip");
  std::memset(&o, 0, sizeof(o));
  o.act_quant = 1;  // int4 weights
  expect(moe_layer_forward_ex(&L, static_cast<uint16_t *>(p), 4, static_cast<float *>(p), nullptr, nullptr, nullptr,
                              p, size_t{1} << 30, &o, nullptr),
         MOE_ERR_UNSUPPORTED, "W8A8 with int4 weights");
  std::memset(&o, 0, sizeof(o));
  o.reserved = 1;
  expect(moe_layer_forward_ex(&L, static_cast<uint16_t *>(p), 4, static_cast<float *>(p), nullptr, nullptr, nullptr,
                              p, size_t{1} << 30, &o, nullptr),
         MOE_ERR_INVALID_ARG, "reserved word");
  moe_residual r;
  std::memset(&r, 0, sizeof(r));
  expect(moe_layer_forward(&L, static_cast<uint16_t *>(p), 4, static_cast<float *>(p), &r, nullptr, nullptr, p,
                           size_t{1} << 30, nullptr),
         MOE_ERR_INVALID_ARG, "residual without buffers");
  expect(moe_layer_forward_noalloc(&L, static_cast<uint16_t *>(p), 0, static_cast<float *>(p), nullptr, nullptr,
                                   nullptr, nullptr, nullptr),
         MOE_OK, "no-alloc T = 0");
  moe_layer bad = L;
  bad.shared.ffn = 256;
  bad.shared_gate_w = static_cast<const float *>(p);
  expect(moe_layer_forward(&bad, static_cast<uint16_t *>(p), 4, static_cast<float *>(p), nullptr, nullptr, nullptr,
                           p, size_t{1} << 30, nullptr) != MOE_OK,
         1, "mismatched shared expert");

  // the other entry points' argument checks
  expect(moe_combine(nullptr, nullptr, 4, 8, 2048, nullptr, nullptr, static_cast<float *>(p), nullptr, nullptr),
         MOE_ERR_INVALID_ARG, "combine without rows");
  expect(moe_combine(static_cast<float *>(p), static_cast<int32_t *>(p), 4, 8, 100, nullptr, nullptr,
                     static_cast<float *>(p), nullptr, nullptr),
         MOE_ERR_INVALID_ARG, "combine H");
  expect(moe_combine(static_cast<float *>(p), static_cast<int32_t *>(p), 0, 8, 2048, nullptr, nullptr,
                     static_cast<float *>(p), nullptr, nullptr),
         MOE_OK, "combine T = 0");
  expect(moe_route(&L, nullptr, 4, static_cast<int32_t *>(p), static_cast<float *>(p), nullptr, nullptr, nullptr, 0,
                   nullptr),
         MOE_ERR_INVALID_ARG, "route without x");
  expect(moe_route(&L, static_cast<uint16_t *>(p), 4, static_cast<int32_t *>(p), static_cast<float *>(p), nullptr,
                   nullptr, nullptr, 0, nullptr),
         MOE_ERR_WORKSPACE, "route without logits or workspace");
  expect(moe_permute(nullptr, nullptr, 4, 8, 256, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                     nullptr, 0, nullptr),
         MOE_ERR_INVALID_ARG, "permute without ids");
  expect(moe_expert_ffn(nullptr, 2048, static_cast<uint16_t *>(p), 4, 32, nullptr, nullptr, nullptr, nullptr,
                        nullptr, static_cast<float *>(p), p, size_t{1} << 30, nullptr),
         MOE_ERR_INVALID_ARG, "expert ffn without weights");
  if (g_fail) {
    std::printf("%d failures\n", g_fail);
    return 1;
  }
  std::printf("ok\n");
  return 0;
}
