"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The HIP sources are built with the sanitizers on their host side only (device
code is compiled as usual and never run here), linked with the C driver
tests/abi_sanitize_main.c, and run on the CPU: every call is refused by argument
validation or is a size query, including sizes at the extremes of their types.
Any sanitizer report, or a return code other than the expected one, fails.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_gqa_amd", "csrc")
SOURCES = ["api", "rope", "store_kvcache", "attn_decode", "attn_prefill", "decode_graph", "sublayer"]
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _tool(*names):
    for n in names:
        p = shutil.which(n) or (n if os.path.exists(n) else None)
        if p:
            return p
    return None


def test_abi_host_code_under_sanitizers(tmp_path):
    hipcc = _tool("hipcc", os.path.join(ROCM, "bin", "hipcc"))
    clang = _tool(os.path.join(ROCM, "lib", "llvm", "bin", "clang"))
    clangxx = _tool(os.path.join(ROCM, "lib", "llvm", "bin", "clang++"))
    if not (hipcc and clang and clangxx):
        pytest.skip("ROCm compilers not available")
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    procs = []
    for s in SOURCES:
        obj = str(tmp_path / f"{s}.o")
        procs.append((s, subprocess.Popen([hipcc, *flags, "-c", os.path.join(CSRC, s + ".hip"), "-o", obj],
                                          stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
    for s, p in procs:
        out, err = p.communicate(timeout=600)
        assert p.returncode == 0, f"hipcc {s}: {err[-2000:]}"
    main_o = str(tmp_path / "main.o")
    subprocess.run([clang, "-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
                    "-I", os.path.join(ROOT, "include"), "-c", os.path.join(ROOT, "tests", "abi_sanitize_main.c"),
                    "-o", main_o], check=True)
    exe = str(tmp_path / "abi_asan")
    subprocess.run([clangxx, "-fsanitize=address,undefined", "-o", exe, main_o,
                    *[str(tmp_path / f"{s}.o") for s in SOURCES],
                    "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib")],
                   check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], env=env, capture_output=True, text=True, timeout=300)
    report = r.stdout + r.stderr
    assert "runtime error" not in report and "AddressSanitizer" not in report, report[-4000:]
    assert r.returncode == 0 and " 0 failures" in r.stdout, report[-4000:]
