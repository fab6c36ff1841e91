"""The allocation-free decode entry point (pkv_attn_decode_paged_noalloc), called
through the C ABI, against the decode entry point that takes a workspace: two calls
in a row, the second on a smaller batch, each byte-identical to the workspace
path on the same inputs and inside the attention gates of the oracle.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import paged_kv_gqa_amd as pkv
import workloads as wl
from gpu_helpers import bits, check_attn, f64, gather_sequences, to_dev

pytestmark = pytest.mark.gpu
D = 128


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pkv.load_library()
    return torch.device("cuda:0")


def _say(*a):
    print("[gpu]", *a, flush=True)


def _noalloc(q, kc, vc, o, cl, bt, hq, hkv):
    lib = pkv.load_library()
    return lib.pkv_attn_decode_paged_noalloc(q.data_ptr(), kc.data_ptr(), vc.data_ptr(), o.data_ptr(), cl.data_ptr(),
                                             bt.data_ptr(), bt.shape[1], q.shape[0], hq, hkv, D, 256, kc.shape[0],
                                             ctypes.c_float(D ** -0.5), torch.cuda.current_stream().cuda_stream)


def _with_workspace(q, kc, vc, o, cl, bt, hq, hkv):
    lib = pkv.load_library()
    need = lib.pkv_attn_decode_workspace_bytes(q.shape[0], hq, hkv, D, bt.shape[1], 256)
    ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    rc = lib.pkv_attn_decode_paged(q.data_ptr(), kc.data_ptr(), vc.data_ptr(), o.data_ptr(), cl.data_ptr(),
                                   bt.data_ptr(), bt.shape[1], q.shape[0], hq, hkv, D, 256, kc.shape[0],
                                   ctypes.c_float(D ** -0.5), ws.data_ptr(), need,
                                   torch.cuda.current_stream().cuda_stream)
    return rc, ws


def test_noalloc_decode_matches_the_workspace_entry_point(dev):
    lib = pkv.load_library()
    # call 1: the Qwen3-8B decode batch (256 sequences, 65 MiB of split-K partials)
    w = wl.paged_decode_8b(seed=0)
    _say("no-alloc decode, call 1: 256 sequences of the 8B workload")
    hq, hkv = 32, 8
    kc = torch.empty((w.num_blocks, 256, hkv, D), dtype=torch.bfloat16, device=dev)
    vc = torch.empty_like(kc)
    wl.fill_normal_bf16_(kc, w.config_id, w.seed, 10)
    wl.fill_normal_bf16_(vc, w.config_id, w.seed, 11)
    q = to_dev(w.q(), dev)
    cl, bt = to_dev(w.context_lens, dev), to_dev(w.block_tables, dev)
    o_na = torch.full((w.batch, hq, D), 7.0, dtype=torch.bfloat16, device=dev)
    o_ws = torch.empty_like(o_na)
    rc = _noalloc(q, kc, vc, o_na, cl, bt, hq, hkv)
    assert rc == 0, lib.pkv_last_error().decode()
    rc, ws = _with_workspace(q, kc, vc, o_ws, cl, bt, hq, hkv)
    assert rc == 0, lib.pkv_last_error().decode()
    torch.cuda.synchronize()
    assert torch.equal(o_na.view(torch.int16), o_ws.view(torch.int16)), "call 1 differs from the workspace path"
    seqs = [0, 1, int(np.argmax(w.context_lens)), int(w.shared_seqs[0])]
    kch, vch, bth = gather_sequences(kc, vc, w.block_tables, seqs, w.context_lens)
    ref = oracle.attn_decode(bits(q)[seqs], kch, vch, w.context_lens[seqs], bth, hq, hkv)
    check_attn(f64(o_na)[seqs], ref, "no-alloc decode, call 1")
    del kc, vc, ws

    # call 2: a smaller batch at other head counts; the array still holds call 1's partials
    _say("no-alloc decode, call 2: 7 sequences, 16/8 heads, ragged contexts (one empty)")
    rng = wl.rng_for(140, 0, 0)
    hq2, hkv2 = 16, 8
    ctx = [1, 255, 256, 3000, 0, 700, 9000]
    mb = max(-(-c // 256) for c in ctx) + 1
    nb = sum(-(-c // 256) for c in ctx) + 2
    perm = rng.permutation(nb)
    rows, nxt = [], 0
    for c in ctx:
        n = -(-c // 256)
        rows.append(list(perm[nxt:nxt + n]))
        nxt += n
    bt2 = wl.pad_block_tables(rows, mb)
    kc2 = wl.normal_bf16(rng, (nb, 256, hkv2, D))
    vc2 = wl.normal_bf16(rng, (nb, 256, hkv2, D))
    q2 = wl.normal_bf16(rng, (len(ctx), hq2, D))
    cl2 = np.array(ctx, np.int32)
    d = [to_dev(x, dev) for x in (q2, kc2, vc2, cl2, bt2)]
    o2_na = torch.full((len(ctx), hq2, D), 7.0, dtype=torch.bfloat16, device=dev)
    o2_ws = torch.empty_like(o2_na)
    rc = _noalloc(d[0], d[1], d[2], o2_na, d[3], d[4], hq2, hkv2)
    assert rc == 0, lib.pkv_last_error().decode()
    rc, _ = _with_workspace(d[0], d[1], d[2], o2_ws, d[3], d[4], hq2, hkv2)
    assert rc == 0, lib.pkv_last_error().decode()
    torch.cuda.synchronize()
    assert torch.equal(o2_na.view(torch.int16), o2_ws.view(torch.int16)), "call 2 differs from the workspace path"
    ref2 = oracle.attn_decode(q2, kc2, vc2, cl2, bt2, hq2, hkv2)
    got2 = f64(o2_na)
    check_attn(got2[cl2 > 0], ref2[cl2 > 0], "no-alloc decode, call 2")
    assert np.all(got2[cl2 == 0] == 0.0)


def test_noalloc_decode_refuses_batches_beyond_its_array(dev):
    """512 sequences with 128-block tables at 32/8 heads need 129 MiB of partials: the call
    returns PKV_ERR_WORKSPACE on the host and launches nothing."""
    _say("no-alloc decode refuses a batch beyond its fixed array")
    lib = pkv.load_library()
    need = lib.pkv_attn_decode_workspace_bytes(512, 32, 8, D, 128, 256)
    assert need > 96 << 20
    t = torch.zeros(16, dtype=torch.int32, device=dev)
    kc = torch.zeros((1, 256, 8, D), dtype=torch.bfloat16, device=dev)
    rc = lib.pkv_attn_decode_paged_noalloc(t.data_ptr(), kc.data_ptr(), kc.data_ptr() + 256,
                                           t.data_ptr(), t.data_ptr(), t.data_ptr(), 128, 512, 32, 8, D, 256, 1,
                                           ctypes.c_float(D ** -0.5), torch.cuda.current_stream().cuda_stream)
    assert rc == -4
    assert "fixed device array" in lib.pkv_last_error().decode()
