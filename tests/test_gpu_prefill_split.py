"""GPU parity of the prefill key split: few query blocks over long key ranges.

When a call's query blocks do not fill the CU slots and its keys run long, the fast
pass cuts each long block's key range into chunks whose partial sums a merge
kernel adds (the call's optional workspace holds them).  These tests run such
calls split and unsplit and compare both with the oracle ("3.3 Model skeleton and
core operators", section 7.2, and "nano-vllm code walkthrough", "Prefill stage":
the same varlen causal attention whatever the launch shape).
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_gqa_amd as pkv
import workloads as wl
from gpu_helpers import bits, check_attn, f64, to_dev

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


def _inputs(dev, lens_q, lens_k, hq, hkv, seed, paged, make_qkv=None):
    """Host arrays and device tensors of one batch; paged batches get a permuted pool."""
    rng = wl.rng_for(95, seed, 0)
    cuq, cuk = wl.cu_seqlens(lens_q), wl.cu_seqlens(lens_k)
    tq, tk = int(cuq[-1]), int(cuk[-1])
    if make_qkv is None:
        q = wl.normal_bf16(rng, (tq, hq, D))
        k = wl.normal_bf16(rng, (tk, hkv, D))
        v = wl.normal_bf16(rng, (tk, hkv, D))
    else:
        q, k, v = make_qkv(rng, tq, tk)
    host = {"q": q, "cuq": cuq, "cuk": cuk, "bt": None}
    d = {"q": to_dev(q, dev), "cuq": to_dev(cuq, dev), "cuk": to_dev(cuk, dev), "bt": None,
         "mq": max(lens_q), "mk": max(lens_k)}
    if not paged:
        host["k"], host["v"] = k, v
        d["k"], d["v"] = to_dev(k, dev), to_dev(v, dev)
        return host, d
    nb = sum(-(-L // 256) for L in lens_k) + 3
    perm = rng.permutation(nb)
    kc = wl.normal_bf16(rng, (nb * 256, hkv, D))
    vc = wl.normal_bf16(rng, (nb * 256, hkv, D))
    rows_bt, nxt, off = [], 0, 0
    for L in lens_k:
        c = -(-L // 256)
        rows_bt.append(list(perm[nxt:nxt + c]))
        nxt += c
    bt = wl.pad_block_tables(rows_bt)
    for b, L in enumerate(lens_k):
        sl = wl.slots_for(bt[b], np.arange(L))
        kc[sl] = k[off:off + L]
        vc[sl] = v[off:off + L]
        off += L
    host.update(k=kc, v=vc, bt=bt)
    d.update(k=to_dev(kc.reshape(nb, 256, hkv, D), dev), v=to_dev(vc.reshape(nb, 256, hkv, D), dev),
             bt=to_dev(bt, dev))
    return host, d


def _call(d, workspace=None, out=None):
    return pkv.attn_prefill_varlen(d["q"], d["k"], d["v"], d["cuq"], d["cuk"], d["mq"], d["mk"],
                                   block_table=d["bt"], out=out, workspace=workspace)


def _rows(lens_q, hq, n, seed):
    """n random (token, head) rows plus every sequence's first and last query on heads 0
    and hq - 1."""
    rng = np.random.default_rng(seed)
    T = sum(lens_q)
    cu = wl.cu_seqlens(lens_q)
    edge = [[int(cu[b]), h] for b in range(len(lens_q)) for h in (0, hq - 1)]
    edge += [[int(cu[b + 1]) - 1, h] for b in range(len(lens_q)) for h in (0, hq - 1)]
    return np.concatenate([np.stack([rng.integers(0, T, n), rng.integers(0, hq, n)], 1), np.array(edge)])


def _oracle(host, hq, hkv, rows):
    return oracle.attn_prefill(host["q"], host["k"], host["v"], host["cuq"], host["cuk"], hq, hkv,
                               block_table=host["bt"], rows=rows)


CASES = [
    # lens_q, lens_k, hq, hkv, paged
    ([256] * 4, [16384] * 4, 32, 8, True),      # later chunks over a long cached context, 4-wave kernel, 2 chunks
    ([256, 256], [8192, 8192], 16, 8, False),   # contiguous K/V with a long prefix, G = 2, 4 chunks
    ([2048], [16384], 8, 2, True),              # 8-wave kernel (mean query length 2048), G = 4, 4 chunks
    ([512, 512], [12288, 9000], 8, 8, True),    # G = 1, unequal contexts (a partial last tile)
    ([128] * 8, [2048] * 8, 32, 8, True),       # 2 chunks, and the 8 units of each XCD dealt as one window
]


@pytest.mark.parametrize("lens_q,lens_k,hq,hkv,paged", CASES)
def test_prefill_split_matches_unsplit_and_oracle(dev, lens_q, lens_k, hq, hkv, paged):
    """Split and unsplit calls both match the oracle; they differ only in the fp32 order
    of the partial sums, so by at most one bf16 step of the output."""
    need = pkv.prefill_workspace_bytes(len(lens_q), sum(lens_q), max(lens_q), max(lens_k), hq, hkv)
    _say(f"prefill split: Lq {lens_q} over Lk {lens_k}, {hq}/{hkv} heads, paged={paged}, workspace {need} B")
    assert need > 0, "this shape is meant to split"
    host, d = _inputs(dev, lens_q, lens_k, hq, hkv, seed=hq + len(lens_q), paged=paged)
    o_split = _call(d)                                              # the binding allocates the workspace
    o_whole = _call(d, workspace=torch.empty(0, dtype=torch.uint8, device=dev))
    torch.cuda.synchronize()
    rows = _rows(lens_q, hq, 400, seed=hq)
    ref = _oracle(host, hq, hkv, rows)
    a, b = f64(o_split), f64(o_whole)
    mx_s, mean_s = check_attn(a[rows[:, 0], rows[:, 1]], ref, "split")
    mx_w, mean_w = check_attn(b[rows[:, 0], rows[:, 1]], ref, "unsplit")
    assert np.isfinite(a).all()
    # The two differ in the fp32 order of the sums over keys.  An output is a sum of
    # thousands of products that largely cancel, so its fp32 error is bounded in
    # absolute terms (the size of the products), not relative to the output: one bf16
    # step of the output plus 2^-14.  A lost or doubled tile would move many outputs
    # by far more, and the error against the oracle with it.
    d = np.abs(a - b)
    bound = np.maximum(np.abs(a), np.abs(b)) * 2.0 ** -7 + 2.0 ** -14
    _say(f"split vs unsplit: max {d.max():.3e}, mean {d.mean():.3e}; oracle max/mean split "
         f"{mx_s:.3e}/{mean_s:.3e}, unsplit {mx_w:.3e}/{mean_w:.3e}")
    assert (d <= bound).all(), f"split vs unsplit: {(d > bound).sum()} outputs beyond the bound, max {d.max():.3e}"
    assert d.mean() <= 2e-5
    assert mean_s <= 1.05 * mean_w + 1e-6


def _extreme(hq, hkv, kind):
    """Some heads' scores leave the fast pass's range: 'large' scales q rows of heads 0
    and hq-1 by 40; 'small' points heads of the first GQA group against a direction
    every key of kv head 0 shares (every score near -100 in base-2 units)."""
    G = hq // hkv

    def make(rng, tq, tk):
        q = wl.bf16_to_f32(wl.normal_bf16(rng, (tq, hq, D))).astype(np.float64)
        k = wl.bf16_to_f32(wl.normal_bf16(rng, (tk, hkv, D))).astype(np.float64)
        v = wl.normal_bf16(rng, (tk, hkv, D))
        if kind == "large":
            q[:, 0] *= 40.0
            q[:, hq - 1] *= 40.0
        else:
            u = rng.choice([-1.0, 1.0], size=D)
            k[:, 0] = u + 0.05 * k[:, 0]
            q[:, :G] = -6.0 * u + 0.5 * q[:, :G]
        return wl.bf16_bits(q), wl.bf16_bits(k), v
    return make


@pytest.mark.parametrize("kind", ["large", "small"])
def test_prefill_split_rows_outside_fast_range(dev, kind):
    """Split items whose summed weights leave the fast pass's range are flagged by the
    merge and recomputed whole by the exact pass."""
    lens_q, lens_k, hq, hkv = [256] * 4, [16384] * 4, 32, 8
    _say(f"prefill split, {kind} scores on some heads")
    host, d = _inputs(dev, lens_q, lens_k, hq, hkv, seed=31, paged=True, make_qkv=_extreme(hq, hkv, kind))
    o = _call(d)
    torch.cuda.synchronize()
    T = sum(lens_q)
    t = np.arange(0, T, 5)
    rows = np.concatenate([np.stack([t, np.zeros_like(t)], 1), np.stack([t, np.full_like(t, hq - 1)], 1),
                           np.stack([t, (t // 5) % hq], 1)])
    ref = _oracle(host, hq, hkv, rows)
    got = f64(o)[rows[:, 0], rows[:, 1]]
    assert np.isfinite(got).all()
    check_attn(got, ref, f"split, {kind} scores")


def test_prefill_split_short_workspace_runs_unsplit(dev):
    """A workspace smaller than the planned size: the call runs unsplit (byte-identical
    to an explicit unsplit call)."""
    lens_q, lens_k, hq, hkv = [256, 256], [8192, 8192], 16, 8
    need = pkv.prefill_workspace_bytes(2, 512, 256, 8192, hq, hkv)
    _say(f"prefill split: workspace of {need - 256} B for {need} needed")
    host, d = _inputs(dev, lens_q, lens_k, hq, hkv, seed=41, paged=False)
    short = torch.empty(need - 256, dtype=torch.uint8, device=dev)
    o1 = _call(d, workspace=short)
    o2 = _call(d, workspace=torch.empty(0, dtype=torch.uint8, device=dev))
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_prefill_split_captured_in_a_graph(dev):
    """A split call (fast pass, merge, exact pass) captured into a HIP graph with its
    workspace and replayed several times, with eager split calls on other workspaces
    between the replays: every replay gives the eager result byte for byte."""
    lens_q, lens_k, hq, hkv = [256] * 4, [16384] * 4, 32, 8
    _say("prefill split captured into a graph and replayed")
    host, d = _inputs(dev, lens_q, lens_k, hq, hkv, seed=47, paged=True, make_qkv=_extreme(hq, hkv, "large"))
    need = pkv.prefill_workspace_bytes(4, 1024, 256, 16384, hq, hkv)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    eager = _call(d)
    torch.cuda.synchronize()
    go = torch.empty_like(eager)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _call(d, workspace=ws, out=go)
    torch.cuda.synchronize()
    for rep in range(3):
        go.fill_(0)
        ws.fill_(0xFF)                   # stale workspace contents must not matter
        g.replay()
        extra = _call(d)
        torch.cuda.synchronize()
        assert torch.equal(go.view(torch.int16), eager.view(torch.int16)), f"replay {rep}"
        assert torch.equal(extra.view(torch.int16), eager.view(torch.int16)), f"replay {rep}: eager call"
