"""The oracle's own safety: it refuses inputs whose keys do not exist instead of
reading outside its arrays, and its C code runs clean under AddressSanitizer and
UndefinedBehaviorSanitizer (a host-only gcc build of oracle/pkv_oracle.c driven by
tests/oracle_sanitize_main.c).
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
D = 128


def _paged_inputs(rng, nb=6, hkv=2):
    kc = wl.normal_bf16(rng, (nb * 256, hkv, D))
    vc = wl.normal_bf16(rng, (nb * 256, hkv, D))
    return kc, vc


@pytest.mark.parametrize("bad", [-1, 6, 1 << 20])
def test_prefill_refuses_unusable_block_ids_inside_a_context(bad):
    rng = wl.rng_for(120, 0, 0)
    kc, vc = _paged_inputs(rng)
    q = wl.normal_bf16(rng, (20, 4, D))
    cuq = np.array([0, 10, 20], np.int32)
    cuk = np.array([0, 300, 700], np.int32)
    bt = np.array([[0, 1, -1], [2, 3, 4]], np.int32)
    oracle.attn_prefill(q, kc, vc, cuq, cuk, 4, 2, block_table=bt)          # -1 past the context: fine
    bt_bad = bt.copy()
    bt_bad[1, 1] = bad
    with pytest.raises(ValueError, match="do not exist"):
        oracle.attn_prefill(q, kc, vc, cuq, cuk, 4, 2, block_table=bt_bad)
    with pytest.raises(ValueError, match="do not exist"):                  # a table too narrow
        oracle.attn_prefill(q, kc, vc, cuq, np.array([0, 300, 1100], np.int32), 4, 2, block_table=bt)


def test_prefill_refuses_contiguous_keys_past_the_end():
    rng = wl.rng_for(121, 0, 0)
    q = wl.normal_bf16(rng, (30, 4, D))
    k = wl.normal_bf16(rng, (30, 2, D))
    cu = np.array([0, 12, 30], np.int32)
    oracle.attn_prefill(q, k, k, cu, cu, 4, 2)
    with pytest.raises(ValueError):
        oracle.attn_prefill(q, k[:29], k[:29], cu, cu, 4, 2)


@pytest.mark.parametrize("bad", [-1, 6])
def test_decode_refuses_unusable_block_ids_inside_a_context(bad):
    rng = wl.rng_for(122, 0, 0)
    kc, vc = _paged_inputs(rng)
    q = wl.normal_bf16(rng, (2, 4, D))
    bt = np.array([[5, -1, -1], [0, 1, 2]], np.int32)
    ctx = np.array([256, 600], np.int32)
    oracle.attn_decode(q, kc, vc, ctx, bt, 4, 2)
    bt_bad = bt.copy()
    bt_bad[1, 2] = bad
    with pytest.raises(ValueError, match="outside the pool"):
        oracle.attn_decode(q, kc, vc, ctx, bt_bad, 4, 2)
    # the same table is fine for a context that stops before the bad entry
    oracle.attn_decode(q, kc, vc, np.array([256, 512], np.int32), bt_bad, 4, 2)


def test_oracle_runs_clean_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    exe = tmp_path / "oracle_sanitize"
    cmd = [gcc, "-O1", "-g", "-std=c11", "-D_GNU_SOURCE", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           os.path.join(ROOT, "tests", "oracle_sanitize_main.c"), os.path.join(ROOT, "oracle", "pkv_oracle.c"),
           "-lm", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
