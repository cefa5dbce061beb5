"""AddressSanitizer and UndefinedBehaviorSanitizer builds on the CPU: the
oracle (every entry point, both weight formats, every variant) and the host
side of the C ABI (argument validation, workspace sizing, status text: every
path that returns before a device is touched).  The GPU code itself is not
instrumented (no sanitizer runs on the device); only host code is."""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "mixture_experts_decode_moe_amd", "csrc")
BUILD = os.path.join(ROOT, "mixture_experts_decode_moe_amd", "_build")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


@pytest.mark.skipif(shutil.which("g++") is None, reason="no g++")
def test_oracle_under_address_and_undefined_behavior_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_check")
    _run(["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", f"-I{os.path.join(ROOT, 'oracle')}", os.path.join(SAN, "oracle_check.cpp"),
          os.path.join(ROOT, "oracle", "moe_oracle.cpp"), "-o", exe, "-lpthread"])
    r = _run([exe], env={**os.environ, "ASAN_OPTIONS": "detect_leaks=1:abort_on_error=0",
                         "UBSAN_OPTIONS": "print_stacktrace=1"})
    assert r.stdout.strip().endswith("ok")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="no hipcc")
def test_host_abi_under_address_sanitizer(tmp_path):
    """The host translation units of the library built with AddressSanitizer
    (each -fsanitize flag behind -Xarch_host: host code only), linked with
    the regular device objects, then driven from a sanitized C++ caller."""
    objs = sorted(glob.glob(os.path.join(BUILD, "*.o")))
    host_units = ("api.o", "noalloc.o")
    if len([o for o in objs if os.path.basename(o) not in host_units]) < 7:
        from mixture_experts_decode_moe_amd import build
        build.build()
        objs = sorted(glob.glob(os.path.join(BUILD, "*.o")))
    flags = ["-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
    san_objs = []
    for unit in host_units:
        out = str(tmp_path / unit)
        _run([HIPCC, *flags, "-c", os.path.join(CSRC, unit.replace(".o", ".hip")), "-o", out])
        san_objs.append(out)
    lib = str(tmp_path / "libmoe_asan.so")
    _run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address",
          "-Xarch_host", "-shared-libasan", *san_objs,
          *[o for o in objs if os.path.basename(o) not in host_units], "-o", lib])
    exe = str(tmp_path / "host_abi_check")
    _run([CLANG, "-std=c++17", "-O1", "-g", "-fsanitize=address", "-shared-libasan", "-fno-omit-frame-pointer",
          f"-I{os.path.join(ROOT, 'include')}", os.path.join(SAN, "host_abi_check.cpp"), f"-L{tmp_path}",
          "-lmoe_asan", f"-Wl,-rpath,{tmp_path}", "-o", exe])
    rt = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    assert rt, "no clang AddressSanitizer runtime"
    env = {**os.environ, "ASAN_OPTIONS": "detect_leaks=0",
           "LD_LIBRARY_PATH": os.path.dirname(rt[0]) + ":" + os.environ.get("LD_LIBRARY_PATH", "")}
    r = _run([exe], env=env)
    assert r.stdout.strip().endswith("ok")
