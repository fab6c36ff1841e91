"""C ABI checks that need no GPU: the library loads, exports every declared
symbol, and rejects invalid arguments on the host before any HIP call."""
import ctypes
import os
import re

import pytest

import paged_kv_gqa_amd as pkv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    with open(os.path.join(ROOT, "include", "pkv.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"PKV_API\s+[\w\s\*]+?\b(pkv_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pkv.LIB_PATH):
        pytest.skip("libpkv.so not built (run python -m paged_kv_gqa_amd.build)")
    return pkv.load_library()


def test_header_declares_the_four_steps():
    syms = _declared_symbols()
    for s in ("pkv_qk_norm_rope", "pkv_store_kvcache", "pkv_attn_prefill_varlen", "pkv_attn_decode_paged"):
        assert s in syms
    assert sorted(pkv.EXPORTED) == syms


def test_library_exports_every_declared_symbol(lib):
    for s in _declared_symbols():
        assert hasattr(lib, s), s
    assert lib.pkv_version() >> 16 == 1


FAKE = ctypes.c_void_p(0x1000)     # never dereferenced: validation fails first


def _err(lib):
    return lib.pkv_last_error().decode()


def test_qk_norm_rope_validation(lib):
    f = lib.pkv_qk_norm_rope
    # Hq not a multiple of Hkv
    assert f(FAKE, 2048, FAKE, 1024, FAKE, FAKE, FAKE, 4, 12, 8, 128, FAKE, FAKE, 1e-6, FAKE, 40960, None) == -1
    assert "multiple" in _err(lib)
    # head_dim other than 128
    assert f(FAKE, 2048, FAKE, 1024, FAKE, FAKE, FAKE, 4, 16, 8, 64, FAKE, FAKE, 1e-6, FAKE, 40960, None) == -2
    # row stride shorter than the row
    assert f(FAKE, 1024, FAKE, 1024, FAKE, FAKE, FAKE, 4, 16, 8, 128, FAKE, FAKE, 1e-6, FAKE, 40960, None) == -1
    # null pointer
    assert f(None, 2048, FAKE, 1024, FAKE, FAKE, FAKE, 4, 16, 8, 128, FAKE, FAKE, 1e-6, FAKE, 40960, None) == -1
    # negative token count; zero tokens is a no-op success
    assert f(FAKE, 2048, FAKE, 1024, FAKE, FAKE, FAKE, -1, 16, 8, 128, FAKE, FAKE, 1e-6, FAKE, 40960, None) == -1
    assert f(None, 2048, None, 1024, None, None, None, 0, 16, 8, 128, None, None, 1e-6, None, 40960, None) == 0
    # in place with a strided input is refused
    assert f(FAKE, 4096, FAKE, 4096, FAKE, ctypes.c_void_p(0x2000), FAKE, 4, 16, 8, 128, FAKE, FAKE, 1e-6, FAKE,
             40960, None) == -1


def test_store_kvcache_validation(lib):
    f = lib.pkv_store_kvcache
    ok_args = [FAKE, 1024, FAKE, 1024, FAKE, ctypes.c_void_p(0x2000), 2048, FAKE, 4, 8, 128, 2, None]
    bad = list(ok_args); bad[1] = 512        # key stride < D
    assert f(*bad) == -1 and "stride" in _err(lib)
    bad = list(ok_args); bad[11] = 3         # element size
    assert f(*bad) == -1
    bad = list(ok_args); bad[7] = None       # slot_mapping missing
    assert f(*bad) == -1
    bad = list(ok_args); bad[5] = FAKE       # k_cache == v_cache
    assert f(*bad) == -1
    bad = list(ok_args); bad[8] = 0          # zero tokens: nothing to do
    assert f(*bad) == 0


def test_prefill_validation(lib):
    f = lib.pkv_attn_prefill_varlen
    o_fake = FAKE.value + (1 << 32)          # an output buffer away from q
    base = [FAKE, 4096, FAKE, 4096, FAKE, 4096, o_fake, FAKE, FAKE, 2, 337, 300, 300, 16, 8, 128, 0.088, 1, None, 0,
            256, 0, None, 0, None]
    a = list(base); a[17] = 0                # causal = 0 is not built
    assert f(*a) == -2
    a = list(base); a[13] = 12               # Hq % Hkv
    assert f(*a) == -1
    a = list(base); a[11] = 400              # max_seqlen_q > max_seqlen_k
    assert f(*a) == -1
    a = list(base); a[18] = FAKE; a[19] = 2; a[21] = 8   # paged with strided k/v rows
    assert f(*a) == -1 and "caches" in _err(lib)
    a = list(base); a[18] = FAKE; a[3] = a[5] = 1024; a[19] = 2; a[20] = 128; a[21] = 8   # block size 128
    assert f(*a) == -2
    a = list(base); a[3] = (1 << 24) + 8      # k row stride beyond 2^24 elements
    assert f(*a) == -1 and "2^24" in _err(lib)
    a = list(base); a[6] = FAKE.value + 4096 * 2 * 336   # o starting inside q's last row
    assert f(*a) == -1 and "overlap" in _err(lib)
    a = list(base); a[0] = 1 << 34; a[6] = (1 << 34) - 337 * 16 * 128 * 2 + 16   # o ending 8 elements into q
    assert f(*a) == -1 and "overlap" in _err(lib)
    a = list(base); a[9] = 0                 # no sequences: no-op
    assert f(*a) == 0
    a = list(base); a[22] = ctypes.c_void_p(o_fake + (1 << 30) + 16); a[23] = 1 << 20   # misaligned workspace
    assert f(*a) == -4 and "aligned" in _err(lib)
    a = list(base); a[22] = ctypes.c_void_p(o_fake); a[23] = 1 << 20   # workspace on top of o
    assert f(*a) == -4 and "overlap" in _err(lib)
    paged = list(base); paged[18] = FAKE; paged[3] = paged[5] = 1024; paged[19] = 2; paged[21] = 8
    cache_end = FAKE.value + 8 * 256 * 1024 * 2
    a = list(paged); a[22] = ctypes.c_void_p(cache_end - 256); a[23] = 1 << 20   # workspace over the caches' tail
    assert f(*a) == -4 and "caches" in _err(lib)
    a = list(base); a[22] = ctypes.c_void_p(((1 << 64) - (1 << 20)) & ~255); a[23] = 2 << 20   # wraps
    assert f(*a) == -4 and "wraps" in _err(lib)


def test_prefill_workspace_query(lib):
    """The key split is planned only for few query blocks over long keys, and the query
    agrees with the binding's arguments (0 for invalid sizes)."""
    ws = lib.pkv_attn_prefill_workspace_bytes
    # 4 x 256 queries over 16384 keys at 32/8 heads: 128 blocks for 512 slots -> a split
    n = ws(4, 1024, 256, 16384, 32, 8, 128)
    assert n > 0 and n % 4 == 0 and n <= 512 << 20
    assert ws(16, 32768, 2048, 4096, 32, 8, 128) == 0      # the 8B prefix batch: many blocks
    assert ws(8, 7316, 1736, 1736, 16, 8, 128) == 0        # the 0.6B varlen batch
    assert ws(4, 1024, 256, 512, 32, 8, 128) == 0          # short keys
    assert ws(4, 1024, 256, 16384, 32, 8, 64) == 0         # head_dim
    assert ws(4, 1024, 256, 16384, 12, 8, 128) == 0        # Hq % Hkv
    assert ws(4, 1024, 300, 200, 32, 8, 128) == 0          # max_seqlen_q > max_seqlen_k


def test_decode_validation_and_workspace(lib):
    ws = lib.pkv_attn_decode_workspace_bytes
    assert ws(64, 16, 8, 128, 32, 256) > 0
    assert ws(64, 16, 8, 64, 32, 256) == 0          # head_dim
    assert ws(64, 12, 8, 128, 32, 256) == 0         # Hq % Hkv
    f = lib.pkv_attn_decode_paged
    need = ws(4, 32, 8, 128, 16, 256)
    base = [FAKE, FAKE, ctypes.c_void_p(0x2000), FAKE, FAKE, FAKE, 16, 4, 32, 8, 128, 256, 100, 0.088,
            ctypes.c_void_p(0x10000), need, None]
    a = list(base); a[15] = need - 1                 # workspace too small
    assert f(*a) == -4
    a = list(base); a[14] = ctypes.c_void_p(0x10010)  # misaligned workspace
    assert f(*a) == -4
    a = list(base); a[11] = 16                        # block size
    assert f(*a) == -2
    a = list(base); a[8] = 24                         # group of 3
    assert f(*a) == -2
    a = list(base); a[12] = 0                         # empty pool
    assert f(*a) == -1
    a = list(base); a[7] = 0                          # empty batch
    assert f(*a) == 0
    far = ctypes.c_void_p(1 << 40)                    # q, caches and o away from the workspace
    ok = [far, ctypes.c_void_p((1 << 40) + (1 << 30)), ctypes.c_void_p((1 << 40) + (2 << 30)),
          ctypes.c_void_p((1 << 40) + (3 << 30))] + base[4:]
    a = list(ok); a[14] = ctypes.c_void_p((1 << 40) + (1 << 30) + (1 << 20))   # inside k_cache
    assert f(*a) == -4 and "overlap" in _err(lib)
    a = list(ok); a[14] = ctypes.c_void_p(((1 << 40) + (3 << 30) - 256))      # running into o
    assert f(*a) == -4 and "overlap" in _err(lib)


def test_qk_norm_rope_store_validation(lib):
    f = lib.pkv_qk_norm_rope_store
    # q, qs, k, ks, v, vs, q_out, k_out, k_cache, v_cache, num_slots, slot, pos, n, Hq, Hkv, d, gq, gk, eps, tab, maxpos
    base = [FAKE, 6144, FAKE, 6144, FAKE, 6144, FAKE, None, ctypes.c_void_p(0x2000), ctypes.c_void_p(0x3000), 4096,
            FAKE, FAKE, 4, 32, 8, 128, FAKE, FAKE, 1e-6, FAKE, 40960, None]
    a = list(base); a[5] = 512               # v stride shorter than the row
    assert f(*a) == -1 and "stride" in _err(lib)
    a = list(base); a[9] = a[8]              # k_cache == v_cache
    assert f(*a) == -1 and "distinct" in _err(lib)
    a = list(base); a[11] = None             # slot_mapping missing
    assert f(*a) == -1
    a = list(base); a[4] = ctypes.c_void_p(0x1008)   # misaligned v
    assert f(*a) == -1 and "aligned" in _err(lib)
    a = list(base); a[16] = 64               # head_dim
    assert f(*a) == -2
    a = list(base); a[10] = -1               # negative pool size
    assert f(*a) == -1
    a = list(base); a[7] = a[2]              # in place k with a strided k
    assert f(*a) == -1 and "in-place" in _err(lib)
    a = list(base); a[13] = 0                # zero tokens: nothing to do
    assert f(*a) == 0


def test_decode_step_desc_layout_matches_c(tmp_path):
    """The ctypes mirror of pkv_decode_step_desc has the C compiler's offsets and size."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    fields = [f for f, _ in pkv.DecodeStepDesc._fields_]
    src = tmp_path / "layout.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "pkv.h"\nint main(void) {\n'
                   + "".join(f'  printf("%zu\\n", offsetof(pkv_decode_step_desc, {f}));\n' for f in fields)
                   + '  printf("%zu\\n", sizeof(pkv_decode_step_desc));\n  return 0;\n}\n')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()]
    want = [getattr(pkv.DecodeStepDesc, f).offset for f in fields] + [ctypes.sizeof(pkv.DecodeStepDesc)]
    assert got == want


def _desc(**kw):
    d = pkv.DecodeStepDesc(qkv=0x1000, qkv_row_stride=6144, q_out=0x2000, o=0x3000, k_cache=0x4000, v_cache=0x5000,
                           num_blocks=64, positions=0x6000, slot_mapping=0x7000, context_lens=0x8000,
                           block_table=0x9000, max_blocks_per_seq=8, max_batch=32, q_norm_weight=0xa000,
                           k_norm_weight=0xb000, cos_sin_cache=0xc000, max_position=40960, eps=1e-6, num_q_heads=32,
                           num_kv_heads=8, head_dim=128, block_size=256, softmax_scale=0.088, flags=0,
                           workspace=0x100000, workspace_bytes=1 << 30)
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def test_decode_graph_validation(lib):
    need = lib.pkv_decode_step_workspace_bytes(32, 32, 8, 128, 8, 256)
    assert need >= max(lib.pkv_attn_decode_workspace_bytes(b, 32, 8, 128, 8, 256) for b in range(1, 33))
    assert lib.pkv_decode_step_workspace_bytes(0, 32, 8, 128, 8, 256) == 0
    d = _desc()
    assert lib.pkv_decode_step(ctypes.byref(d), 33, None) == -1          # batch > max_batch
    assert lib.pkv_decode_step(ctypes.byref(d), 0, None) == 0            # empty step
    small = _desc(workspace_bytes=need - 1)
    assert lib.pkv_decode_step(ctypes.byref(small), 1, None) == -4       # workspace short for some batch size
    assert lib.pkv_decode_step(ctypes.byref(_desc(qkv_row_stride=4096)), 1, None) == -1
    h = ctypes.c_void_p(123)
    bad = (ctypes.c_int32 * 3)(1, 4, 4)                                   # not strictly increasing
    assert lib.pkv_decode_graph_create(ctypes.byref(d), bad, 3, ctypes.byref(h)) == -1 and h.value is None
    big = (ctypes.c_int32 * 2)(16, 64)                                    # beyond max_batch
    assert lib.pkv_decode_graph_create(ctypes.byref(d), big, 2, ctypes.byref(h)) == -1
    assert lib.pkv_decode_graph_bucket(None, 3) == -1
    assert lib.pkv_decode_graph_launch(None, 3, None) == -1
    lib.pkv_decode_graph_destroy(None)


def test_sublayer_ops_validation(lib):
    R = ctypes.c_void_p(0x2000)
    f = lib.pkv_add_rms_norm
    assert f(FAKE, R, FAKE, FAKE, ctypes.c_void_p(0x4000), 4, 4100, 1e-6, None) == -1       # hidden % 8
    assert f(FAKE, R, FAKE, FAKE, ctypes.c_void_p(0x4000), 4, 32768, 1e-6, None) == -2      # above 16384
    assert f(FAKE, R, FAKE, FAKE, None, 4, 4096, 1e-6, None) == -1                          # residual without output
    assert f(FAKE, None, FAKE, FAKE, R, 4, 4096, 1e-6, None) == -1                          # output without residual
    assert f(FAKE, R, FAKE, R, R, 4, 4096, 1e-6, None) == -1 and "differ" in _err(lib)       # y == residual_out
    assert f(ctypes.c_void_p(0x1008), R, FAKE, FAKE, ctypes.c_void_p(0x4000), 4, 4096, 1e-6, None) == -1
    assert f(None, None, None, None, None, 0, 4096, 1e-6, None) == 0                         # empty
    g = lib.pkv_silu_and_mul
    assert g(FAKE, 24576, R, 12288, 4, 12300, None) == -1                                    # intermediate % 8
    assert g(FAKE, 12288, R, 12288, 4, 12288, None) == -1                                    # x rows too short
    assert g(FAKE, 24576, R, 12280, 4, 12288, None) == -1                                    # out rows too short
    assert g(FAKE, 24576, None, 12288, 4, 12288, None) == -1
    assert g(None, 24576, None, 12288, 0, 12288, None) == 0
    h = lib.pkv_sample_gumbel
    T, TOK = ctypes.c_void_p(0x5000), ctypes.c_void_p(0x6000)
    assert h(FAKE, 151936, 2, T, None, 0, 1, 0, TOK, 4, 151936, None) == -2                  # dtype
    assert h(FAKE, 151930, 0, T, None, 0, 1, 0, TOK, 4, 151936, None) == -1                  # stride < vocab
    assert h(FAKE, 151939, 0, T, None, 0, 1, 0, TOK, 4, 151936, None) == -1                  # bf16 stride % 8
    assert h(FAKE, 151936, 0, T, R, 151935, 1, 0, TOK, 4, 151936, None) == -1                # noise stride
    assert h(FAKE, 151936, 0, None, None, 0, 1, 0, TOK, 4, 151936, None) == -1               # temperatures
    assert h(None, 151936, 0, None, None, 0, 1, 0, None, 0, 151936, None) == 0               # no rows


def test_binding_refuses_mismatched_metadata_before_any_call(lib):
    """The Python binding checks metadata counts and where tensors live before it passes
    pointers on: a short cu_seqlens_k, a block table with fewer rows than sequences, a
    context-length vector of the wrong size, or host tensors, raise ValueError."""
    import torch
    bf = torch.bfloat16
    q = torch.zeros((10, 4, 128), dtype=bf)
    k = torch.zeros((10, 2, 128), dtype=bf)
    cu2 = torch.tensor([0, 4, 10], dtype=torch.int32)
    with pytest.raises(ValueError, match="cu_seqlens_k"):
        pkv.attn_prefill_varlen(q, k, k, cu2, torch.tensor([0, 10], dtype=torch.int32), 6, 6)
    kc = torch.zeros((3, 256, 2, 128), dtype=bf)
    with pytest.raises(ValueError, match="block_table"):
        pkv.attn_prefill_varlen(q, kc, kc, cu2, cu2, 6, 6, block_table=torch.zeros((1, 3), dtype=torch.int32))
    with pytest.raises(ValueError, match="GPU"):
        pkv.attn_prefill_varlen(q, k, k, cu2, cu2, 6, 6)
    qd = torch.zeros((3, 4, 128), dtype=bf)
    with pytest.raises(ValueError, match="cache_seqlens"):
        pkv.attn_decode_paged(qd, kc, kc, torch.zeros(2, dtype=torch.int32), torch.zeros((3, 2), dtype=torch.int32))
    with pytest.raises(ValueError, match="cache_seqlens"):
        pkv.attn_decode_paged(qd, kc, kc, torch.zeros(3, dtype=torch.int32), torch.zeros((2, 2), dtype=torch.int32))
    with pytest.raises(ValueError, match="GPU"):
        pkv.attn_decode_paged(qd, kc, kc, torch.zeros(3, dtype=torch.int32), torch.zeros((3, 2), dtype=torch.int32))
    with pytest.raises(ValueError, match="same number"):
        pkv.store_kvcache(k, k[:5], kc, kc, torch.zeros(10, dtype=torch.int32))
