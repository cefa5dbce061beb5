"""The C-ABI library without a GPU: it loads, exports every entry point the
header declares, and rejects bad arguments before anything is launched."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def mb():
    from mixture_experts_decode_moe_amd import binding
    return binding


def test_header_declares_the_entry_points():
    names = declared_functions()
    for required in ("moe_route", "moe_permute", "moe_expert_ffn", "moe_combine", "moe_layer_forward",
                     "moe_workspace_bytes", "moe_status_string"):
        assert required in names


def test_library_exports_every_declared_symbol(mb):
    lib = ctypes.CDLL(mb.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in moe.h but not exported"
    assert set(declared_functions()) <= set(mb.EXPORTED) | {"moe_workspace_init"}


def test_status_strings(mb):
    assert mb.status_string(0) == "ok"
    for s in (-1, -2, -3, -4):
        assert mb.status_string(s) not in ("ok", "unknown status")
    assert mb.status_string(7) == "unknown status"


def _fake_layer(mb, H=2048, E=256, K=8, F=512, fmt=2, shared=True):
    p = ctypes.c_void_p(1 << 20)  # aligned, never dereferenced by the host-only calls
    ex = mb.MoeExperts(fmt, E, F, 0, p, p, p, p, p, p)
    sh = mb.MoeExperts(fmt, 1, F, 0, p, p, p, p, p, p) if shared else mb.MoeExperts()
    return mb.MoeLayer(H, E, K, 1, p, None, ex, sh)


def test_workspace_bytes_is_pure_and_grows(mb):
    lib = mb.raw_lib()
    L = _fake_layer(mb)
    a = lib.moe_workspace_bytes(ctypes.byref(L), 1)
    b = lib.moe_workspace_bytes(ctypes.byref(L), 16)
    c = lib.moe_workspace_bytes(ctypes.byref(L), 2048)
    assert 0 < a < b < c and c % 256 == 0
    assert lib.moe_workspace_bytes(ctypes.byref(L), -1) == 0
    assert lib.moe_permute_workspace_bytes(2048, 8, 256) >= 2048 * 8 * 4
    assert lib.moe_expert_ffn_workspace_bytes(10, 512) >= 10 * 512 * 4


@pytest.mark.parametrize("mutate,expect", [
    (lambda L: setattr(L, "top_k", 0), -1),
    (lambda L: setattr(L, "top_k", 300), -1),
    (lambda L: setattr(L, "renorm", 2), -1),
    (lambda L: setattr(L, "n_experts", 2048), -2),
    (lambda L: setattr(L, "hidden", 1000), -2),
    (lambda L: setattr(L.routed, "fmt", 9), -2),
    (lambda L: setattr(L.routed, "n_experts", 7), -1),
    (lambda L: setattr(L.routed, "ffn", 500), -2),
    (lambda L: setattr(L.routed, "gate_q", None), -1),
    (lambda L: setattr(L.routed, "reserved", 1), -1),
    (lambda L: setattr(L.shared, "n_experts", 2), -1),
    (lambda L: setattr(L, "router_w", None), -1),
    (lambda L: setattr(L, "shared_gate_w", (1 << 20) + 4), -1),  # a gate row not 16-byte aligned
])
def test_layer_validation_rejects_before_launch(mb, mutate, expect):
    lib = mb.raw_lib()
    L = _fake_layer(mb)
    mutate(L)
    p = ctypes.c_void_p(1 << 20)
    rc = lib.moe_layer_forward(ctypes.byref(L), p, 4, p, None, None, None, p, 1 << 30, None)
    assert rc == expect
    assert lib.moe_workspace_bytes(ctypes.byref(L), 4) == 0


def test_other_entry_points_reject_bad_arguments(mb):
    lib = mb.raw_lib()
    p = ctypes.c_void_p(1 << 20)
    assert lib.moe_layer_forward(None, p, 4, p, None, None, None, p, 1 << 30, None) == -1
    L = _fake_layer(mb)
    assert lib.moe_layer_forward(ctypes.byref(L), p, -1, p, None, None, None, p, 1 << 30, None) == -1
    assert lib.moe_layer_forward(ctypes.byref(L), p, 0, p, None, None, None, p, 1 << 30, None) == 0
    assert lib.moe_layer_forward(ctypes.byref(L), p, 4, p, None, None, None, None, 0, None) == -3
    assert lib.moe_layer_forward(ctypes.byref(L), p, 4, p, None, None, None, p, 16, None) == -3
    assert lib.moe_layer_forward(ctypes.byref(L), ctypes.c_void_p((1 << 20) + 2), 4, p, None, None, None, p,
                                 1 << 30, None) == -1
    assert lib.moe_route(ctypes.byref(L), p, 4, None, p, p, None, None, 0, None) == -1
    # logits optional: without them the call needs a workspace for them
    assert lib.moe_route(ctypes.byref(L), p, 4, p, p, None, None, None, 0, None) == -3
    assert lib.moe_route(ctypes.byref(L), p, 4, p, p, None, None, p, 16, None) == -3
    assert lib.moe_route_workspace_bytes(ctypes.byref(L), 4) >= 4 * 256 * 4
    assert lib.moe_route_workspace_bytes(ctypes.byref(L), -1) == 0
    # batches above 16 tokens: the router GEMM's partial sums also pass
    # through the workspace, so it is needed even with logits given
    assert lib.moe_route_workspace_bytes(ctypes.byref(L), 64) >= 64 * 256 * 4 * 5
    assert lib.moe_route(ctypes.byref(L), p, 64, p, p, p, None, None, 0, None) == -3
    assert lib.moe_permute(p, p, 4, 9, 8, p, p, p, p, p, p, p, p, 1 << 20, None) == -1  # K > E
    assert lib.moe_permute(p, p, 4, 2, 4096, p, p, p, p, p, p, p, p, 1 << 20, None) == -2
    assert lib.moe_permute(p, p, 4, 2, 8, p, p, p, p, p, p, p, None, 0, None) == -3
    ex = mb.MoeExperts(2, 256, 512, 0, p, p, p, p, p, p)
    assert lib.moe_expert_ffn(ctypes.byref(ex), 2048, p, 4, 32, None, None, None, p, p, p, p, 1 << 30,
                              None) == -1  # routed set without offsets
    assert lib.moe_combine(p, p, 4, 8, 2046, None, None, p, None, None) == -1
    bad = mb.MoeResidual(None, 1 << 20, None, 1e-6, 0)  # residual_out without residual_in
    assert lib.moe_combine(p, p, 4, 8, 2048, None, None, p, ctypes.byref(bad), None) == -1
    assert lib.moe_layer_forward(ctypes.byref(_fake_layer(mb)), p, 4, p, ctypes.byref(bad), None, None, p,
                                 1 << 30, None) == -1
    assert lib.moe_workspace_init(None, 0, None) == -3


def test_stack_forward_rejects_bad_arguments(mb):
    """moe_stack_forward checks its layers, buffers and workspace before
    launching anything."""
    lib = mb.raw_lib()
    p = ctypes.c_void_p(1 << 20)
    arr = (mb.MoeLayer * 2)(_fake_layer(mb), _fake_layer(mb))
    f = lib.moe_stack_forward
    assert f(None, 2, p, 4, p, p, p, 1e-6, p, None, None, p, 1 << 30, None) == -1
    assert f(arr, 0, p, 4, p, p, p, 1e-6, p, None, None, p, 1 << 30, None) == -1
    assert f(arr, 2, p, 4, None, p, p, 1e-6, p, None, None, p, 1 << 30, None) == -1  # no residual_in
    assert f(arr, 2, p, 4, p, p, None, 1e-6, p, None, None, p, 1 << 30, None) == -1  # no normed_out
    assert f(arr, 2, p, 4, p, p, p, -1.0, p, None, None, p, 1 << 30, None) == -1  # eps < 0
    assert f(arr, 2, p, 0, p, p, p, 1e-6, p, None, None, p, 1 << 30, None) == 0  # no tokens: nothing to do
    assert f(arr, 2, p, 4, p, p, p, 1e-6, p, None, None, None, 0, None) == -3  # no workspace
    assert f(arr, 2, p, 4, p, p, p, 1e-6, p, None, None, p, 16, None) == -3  # too small
    other = _fake_layer(mb)
    other.top_k = 4
    arr2 = (mb.MoeLayer * 2)(_fake_layer(mb), other)
    assert f(arr2, 2, p, 4, p, p, p, 1e-6, p, None, None, p, 1 << 30, None) == -1  # shapes differ


def test_calibration_helpers_reject_bad_arguments(mb):
    """The measurement helpers check their arguments before touching a
    device."""
    lib = mb.raw_lib()
    ms, ops = ctypes.c_float(), ctypes.c_double()
    p = ctypes.c_void_p(1 << 20)
    assert lib.moe_calib_mfma(3, 10, ctypes.byref(ms), ctypes.byref(ops), None) == -1
    assert lib.moe_calib_mfma(0, 0, ctypes.byref(ms), ctypes.byref(ops), None) == -1
    assert lib.moe_calib_mfma(0, 10, None, ctypes.byref(ops), None) == -1
    assert lib.moe_calib_read(None, 1 << 20, ctypes.byref(ms), None) == -1
    assert lib.moe_calib_read(p, 0, ctypes.byref(ms), None) == -1
    assert lib.moe_calib_read(p, 1000, ctypes.byref(ms), None) == -1  # not a multiple of 16
    assert lib.moe_calib_read(ctypes.c_void_p((1 << 20) + 8), 1 << 20, ctypes.byref(ms), None) == -1


def test_forward_options_are_validated(mb):
    """Per-call options: an unknown path or a nonzero reserved word is
    rejected before anything is launched; all-zero options are the
    defaults."""
    lib = mb.raw_lib()
    p = ctypes.c_void_p(1 << 20)
    L = _fake_layer(mb)
    o = mb.forward_opts()
    assert lib.moe_layer_forward_ex(ctypes.byref(L), p, 0, p, None, None, None, p, 1 << 30, ctypes.byref(o),
                                    None) == 0
    o.path = 3
    assert lib.moe_layer_forward_ex(ctypes.byref(L), p, 4, p, None, None, None, p, 1 << 30, ctypes.byref(o),
                                    None) == -1
    o = mb.forward_opts(tail_skip=-1)
    assert lib.moe_layer_forward_ex(ctypes.byref(L), p, 4, p, None, None, None, p, 1 << 30, ctypes.byref(o),
                                    None) == -1
    o = mb.forward_opts(act_quant=2)
    assert lib.moe_layer_forward_ex(ctypes.byref(L), p, 4, p, None, None, None, p, 1 << 30, ctypes.byref(o),
                                    None) == -1
    o = mb.forward_opts(act_quant=1)  # the W8A8 variant needs int8 row-scaled weights
    assert lib.moe_layer_forward_ex(ctypes.byref(L), p, 4, p, None, None, None, p, 1 << 30, ctypes.byref(o),
                                    None) == -2
    o = mb.forward_opts("prefill")
    o.reserved = 5
    assert lib.moe_layer_forward_ex(ctypes.byref(L), p, 4, p, None, None, None, p, 1 << 30, ctypes.byref(o),
                                    None) == -1
    assert mb.forward_opts("decode").path == 1 and mb.forward_opts("prefill").path == 2


def test_no_process_global_mutable_state_in_the_host_code():
    """The host side keeps nothing between calls: no file-scope variables
    (the profiling events are a per-call option), only functions, types and
    constants."""
    src = open(os.path.join(ROOT, "mixture_experts_decode_moe_amd", "csrc", "api.hip")).read()
    src = re.sub(r"//.*", "", src)
    assert "thread_local" not in src
    assert not re.search(r"^static\s+(?!inline|bool|int|size_t|hipError_t|void|const)", src, flags=re.M)
    assert not re.search(r"^(hipEvent_t|int|float|bool)\s+\w+\s*(\[.*\])?\s*(=.*)?;", src, flags=re.M)


def test_shared_gate_needs_a_shared_expert(mb):
    lib = mb.raw_lib()
    p = ctypes.c_void_p(1 << 20)
    L = _fake_layer(mb, shared=False)
    L.shared_gate_w = 1 << 20
    assert lib.moe_workspace_bytes(ctypes.byref(L), 4) == 0
    assert lib.moe_layer_forward(ctypes.byref(L), p, 4, p, None, None, None, p, 1 << 30, None) == -1
    L = _fake_layer(mb, shared=True)
    L.shared_gate_w = 1 << 20
    assert lib.moe_workspace_bytes(ctypes.byref(L), 4) > 0
