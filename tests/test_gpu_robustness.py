"""GPU robustness: bytes the method never reads cannot reach its outputs, outputs are
written exactly where they belong, the fast prefill pass keeps its accuracy for
larger scores, and the kernel's single rounding stays close to the pages' pipeline.

Every expected value comes from ``oracle``; inputs from the seeded generators in
``workloads``.  Gates are in tests/gpu_helpers.py.
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
NAN_BF16 = 0x7FC0


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pkv.load_library()
    return torch.device("cuda:0")


def _say(*a):
    print("[gpu]", *a, flush=True)


def _paged_batch(rng, lens_q, lens_k, hq, hkv, spare_blocks=5):
    """q, a permuted pool holding each sequence's keys, its block table (-1 padded, one
    column wider than needed) and a mask of the cache slots some query can see."""
    cuq, cuk = wl.cu_seqlens(lens_q), wl.cu_seqlens(lens_k)
    need = [-(-L // 256) for L in lens_k]
    nb = sum(need) + spare_blocks
    perm = rng.permutation(nb)
    rows, nxt = [], 0
    for c in need:
        rows.append(list(perm[nxt:nxt + c]))
        nxt += c
    bt = wl.pad_block_tables(rows, max(need) + 1)
    kc = wl.normal_bf16(rng, (nb * 256, hkv, D))
    vc = wl.normal_bf16(rng, (nb * 256, hkv, D))
    q = wl.normal_bf16(rng, (int(cuq[-1]), hq, D))
    used = np.zeros(nb * 256, bool)
    for b, L in enumerate(lens_k):
        used[wl.slots_for(bt[b], np.arange(L))] = True
    return q, kc, vc, cuq, cuk, bt, used


def _prefill(dev, q, kc, vc, cuq, cuk, bt, lens_q, lens_k, hkv, out=None):
    nb = kc.shape[0] // 256
    return pkv.attn_prefill_varlen(to_dev(q, dev), to_dev(kc.reshape(nb, 256, hkv, D), dev),
                                   to_dev(vc.reshape(nb, 256, hkv, D), dev), to_dev(cuq, dev), to_dev(cuk, dev),
                                   max(lens_q), max(lens_k), block_table=to_dev(bt, dev), out=out)


@pytest.mark.parametrize("lens_q,lens_k,hq,hkv", [
    ([40, 257, 1], [300, 513, 1000], 32, 8),                 # one launch of the exact pass, 4 waves
    ([2048], [2300], 4, 1),                                   # one launch, 8 waves (mean query length >= 2048)
    ([1000] * 6, [3000, 2500, 1999, 1000, 3333, 2049], 32, 8),  # fast + exact pass, 4 waves
    ([2048] * 4, [4000, 2048, 3001, 4096], 32, 8),            # fast + exact pass, 8 waves
])
def test_prefill_paged_nan_canaries(dev, lens_q, lens_k, hq, hkv):
    """Case-2 prefill reads keys only through the block table, and only below each
    sequence's Lk: NaN in every other cache slot (the rest of the last block, blocks no
    table lists, what sits behind the -1 padding) leaves the output byte-identical."""
    _say(f"prefill paged NaN canaries: Lq {lens_q}, Lk {lens_k}, {hq}/{hkv} heads")
    rng = wl.rng_for(130, len(lens_q) + hq, 0)
    q, kc, vc, cuq, cuk, bt, used = _paged_batch(rng, lens_q, lens_k, hq, hkv)
    o = _prefill(dev, q, kc, vc, cuq, cuk, bt, lens_q, lens_k, hkv)
    kc2, vc2 = kc.copy(), vc.copy()
    kc2[~used] = NAN_BF16
    vc2[~used] = NAN_BF16
    o2 = _prefill(dev, q, kc2, vc2, cuq, cuk, bt, lens_q, lens_k, hkv)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16)), "bytes outside the contexts changed the output"
    t = np.arange(0, q.shape[0], 11)
    rows = np.stack([t, t % hq], 1)
    ref = oracle.attn_prefill(q, kc, vc, cuq, cuk, hq, hkv, block_table=bt, rows=rows)
    check_attn(f64(o2)[rows[:, 0], rows[:, 1]], ref, "prefill with NaN canaries")


@pytest.mark.parametrize("lens", [[37, 300, 65], [1024] * 8])
def test_prefill_contiguous_nan_past_the_last_row(dev, lens):
    """Case-1 prefill over k/v views whose storage continues with NaN rows after the last
    key: the last partial tile never reads past the end, so the output is unchanged."""
    _say(f"prefill case 1 with NaN rows after the last key, lengths {lens}")
    rng = wl.rng_for(131, len(lens), 0)
    hq, hkv = 16, 8
    T = sum(lens)
    cu = wl.cu_seqlens(lens)
    q = wl.normal_bf16(rng, (T, hq, D))
    k = wl.normal_bf16(rng, (T + 300, hkv, D))
    v = wl.normal_bf16(rng, (T + 300, hkv, D))
    k[T:] = NAN_BF16
    v[T:] = NAN_BF16
    kd, vd = to_dev(k, dev), to_dev(v, dev)
    o = pkv.attn_prefill_varlen(to_dev(q, dev), kd[:T], vd[:T], to_dev(cu, dev), to_dev(cu, dev), max(lens), max(lens))
    torch.cuda.synchronize()
    got = f64(o)
    assert np.isfinite(got).all()
    t = np.arange(0, T, 3)
    rows = np.stack([t, t % hq], 1)
    ref = oracle.attn_prefill(q, k[:T], v[:T], cu, cu, hq, hkv, rows=rows)
    check_attn(got[rows[:, 0], rows[:, 1]], ref, "prefill, NaN after the last key")


def _guarded(shape, dev, fill=0x5A5A, guard=4104):
    """An output view in the middle of a larger buffer whose guard elements hold a pattern
    (4104 elements: the view stays 16-byte aligned, as the kernels require)."""
    n = int(np.prod(shape))
    buf = torch.full((guard + n + guard,), fill, dtype=torch.int16, device=dev)
    return buf, buf[guard:guard + n].view(torch.bfloat16).view(shape), guard


def _guards_intact(buf, guard, n, fill=0x5A5A):
    head = buf[:guard]
    tail = buf[guard + n:]
    return bool(torch.all(head == fill)) and bool(torch.all(tail == fill))


@pytest.mark.parametrize("lens_q,lens_k,paged", [
    ([37, 300], [37, 300], False), ([1024] * 8, [1024] * 8, False),
    ([40, 257], [300, 513], True), ([2048] * 4, [4096] * 4, True)])
def test_prefill_writes_only_its_output_rows(dev, lens_q, lens_k, paged):
    """Guard elements before and after o stay untouched (both launch forms, both loaders)."""
    _say(f"prefill guard bytes around o: Lq {lens_q}, Lk {lens_k}, paged={paged}")
    hq, hkv = 32, 8
    rng = wl.rng_for(132, len(lens_q), int(paged))
    shape = (sum(lens_q), hq, D)
    buf, o, guard = _guarded(shape, dev)
    if paged:
        q, kc, vc, cuq, cuk, bt, _ = _paged_batch(rng, lens_q, lens_k, hq, hkv)
        _prefill(dev, q, kc, vc, cuq, cuk, bt, lens_q, lens_k, hkv, out=o)
        t = np.arange(0, shape[0], 13)
        ref = oracle.attn_prefill(q, kc, vc, cuq, cuk, hq, hkv, block_table=bt, rows=np.stack([t, t % hq], 1))
    else:
        cu = wl.cu_seqlens(lens_q)
        q = wl.normal_bf16(rng, shape)
        k = wl.normal_bf16(rng, (shape[0], hkv, D))
        v = wl.normal_bf16(rng, (shape[0], hkv, D))
        pkv.attn_prefill_varlen(to_dev(q, dev), to_dev(k, dev), to_dev(v, dev), to_dev(cu, dev), to_dev(cu, dev),
                                max(lens_q), max(lens_q), out=o)
        t = np.arange(0, shape[0], 13)
        ref = oracle.attn_prefill(q, k, v, cu, cu, hq, hkv, rows=np.stack([t, t % hq], 1))
    torch.cuda.synchronize()
    assert _guards_intact(buf, guard, o.numel())
    check_attn(f64(o)[t, t % hq], ref, "prefill into a guarded buffer")


def test_decode_writes_only_its_output_and_workspace(dev):
    """Guard elements around o and around the split-K workspace stay untouched."""
    _say("decode guard bytes around o and the workspace")
    rng = wl.rng_for(133, 0, 0)
    hq, hkv = 32, 8
    ctx = [1, 255, 256, 1000, 5000, 0, 33000]
    q, kc, vc, _, _, bt, _ = _paged_batch(rng, [1] * len(ctx), [max(c, 1) for c in ctx], hq, hkv)
    q = wl.normal_bf16(rng, (len(ctx), hq, D))
    cl = np.array(ctx, np.int32)
    nb = kc.shape[0] // 256
    buf, o, guard = _guarded((len(ctx), hq, D), dev)
    need = pkv.decode_workspace_bytes(len(ctx), hq, hkv, bt.shape[1])
    ws_buf = torch.full((4096 + need + 4096,), 0x33, dtype=torch.uint8, device=dev)
    ws = ws_buf[4096:4096 + need]
    pkv.attn_decode_paged(to_dev(q, dev), to_dev(kc.reshape(nb, 256, hkv, D), dev),
                          to_dev(vc.reshape(nb, 256, hkv, D), dev), to_dev(cl, dev), to_dev(bt, dev), out=o,
                          workspace=ws)
    torch.cuda.synchronize()
    assert _guards_intact(buf, guard, o.numel())
    assert bool(torch.all(ws_buf[:4096] == 0x33)) and bool(torch.all(ws_buf[4096 + need:] == 0x33))
    ref = oracle.attn_decode(q, kc, vc, cl, bt, hq, hkv)
    check_attn(f64(o), ref, "decode into a guarded buffer")


def test_qk_norm_rope_outputs_stay_in_bounds(dev):
    """Guard elements around q_out / k_out of the unfused and the fused QK-Norm + RoPE, at
    token counts on both sides of the head-splitting threshold."""
    hq, hkv = 32, 8
    table = pkv.rope_cache_build(40960, D, 1e6, device=dev)
    rng = wl.rng_for(134, 0, 0)
    for n in (1, 7, 256, 3001):
        _say(f"qk_norm_rope guard bytes, {n} tokens")
        qkv = to_dev(wl.normal_bf16(rng, (n, (hq + 2 * hkv) * D)), dev)
        q = qkv[:, :hq * D].view(n, hq, D)
        k = qkv[:, hq * D:(hq + hkv) * D].view(n, hkv, D)
        v = qkv[:, (hq + hkv) * D:].view(n, hkv, D)
        pos = to_dev(rng.integers(0, 40960, n).astype(np.int64), dev)
        g = to_dev(wl.gamma_bf16(rng), dev)
        qb, qo, gq = _guarded((n, hq, D), dev)
        kb, ko, gk = _guarded((n, hkv, D), dev)
        pkv.qk_norm_rope(q, k, pos, g, g, table, 1e-6, q_out=qo, k_out=ko)
        torch.cuda.synchronize()
        assert _guards_intact(qb, gq, qo.numel()) and _guards_intact(kb, gk, ko.numel())
        q_ref, k_ref = qo.clone(), ko.clone()
        kc = torch.zeros((-(-n // 256) + 1, 256, hkv, D), dtype=torch.bfloat16, device=dev)
        vc = torch.zeros_like(kc)
        slots = to_dev(rng.permutation(kc.shape[0] * 256)[:n].astype(np.int32), dev)
        qb2, qo2, gq2 = _guarded((n, hq, D), dev)
        kb2, ko2, gk2 = _guarded((n, hkv, D), dev)
        pkv.qk_norm_rope_store(q, k, v, pos, g, g, table, kc, vc, slots, 1e-6, q_out=qo2, k_out=ko2)
        torch.cuda.synchronize()
        assert _guards_intact(qb2, gq2, qo2.numel()) and _guards_intact(kb2, gk2, ko2.numel())
        assert torch.equal(qo2.view(torch.int16), q_ref.view(torch.int16))
        assert torch.equal(ko2.view(torch.int16), k_ref.view(torch.int16))


def test_binding_refuses_a_wrong_output_buffer(dev):
    """A caller-supplied out of the wrong shape, dtype or layout raises before any launch."""
    _say("binding refuses mis-sized outputs")
    q = torch.zeros((10, 4, D), dtype=torch.bfloat16, device=dev)
    k = torch.zeros((10, 2, D), dtype=torch.bfloat16, device=dev)
    cu = torch.tensor([0, 10], dtype=torch.int32, device=dev)
    for bad in (torch.empty((9, 4, D), dtype=torch.bfloat16, device=dev),
                torch.empty((10, 4, D), dtype=torch.float32, device=dev),
                torch.empty((10, D, 4), dtype=torch.bfloat16, device=dev).transpose(1, 2)):
        with pytest.raises(ValueError, match="out"):
            pkv.attn_prefill_varlen(q, k, k, cu, cu, 10, 10, out=bad)
    kc = torch.zeros((2, 256, 2, D), dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError, match="out"):
        pkv.attn_decode_paged(q[:3].contiguous(), kc, kc, torch.ones(3, dtype=torch.int32, device=dev),
                              torch.zeros((3, 2), dtype=torch.int32, device=dev),
                              out=torch.empty((3, 4, 64), dtype=torch.bfloat16, device=dev))


@pytest.mark.parametrize("lens,paged", [([1024] * 8, False), ([2048] * 4, False), ([1024] * 8, True)])
def test_prefill_fast_pass_with_larger_scores(dev, lens, paged):
    """Batches large enough for the fast pass, q scaled by 3 ... 9 per head (scores of
    roughly 15 to 45 in base-2 units: peaked rows, but sums inside the fast pass's
    window), every row against the oracle."""
    hq, hkv = 16, 8
    _say(f"prefill fast pass with q scaled x3..x9 per head, lengths {lens[:2]}.. ({len(lens)} seqs), paged={paged}")
    rng = wl.rng_for(135, len(lens), int(paged))
    scales = np.linspace(3.0, 9.0, hq).astype(np.float32)
    if paged:
        lens_k = [L + 700 for L in lens]
        q, kc, vc, cuq, cuk, bt, _ = _paged_batch(rng, lens, lens_k, hq, hkv)
        q = wl.bf16_bits(wl.bf16_to_f32(q).reshape(-1, hq, D) * scales[None, :, None])
        o = _prefill(dev, q, kc, vc, cuq, cuk, bt, lens, lens_k, hkv)
        ref = oracle.attn_prefill(q, kc, vc, cuq, cuk, hq, hkv, block_table=bt)
    else:
        T = sum(lens)
        cu = wl.cu_seqlens(lens)
        q = wl.bf16_bits(rng.standard_normal((T, hq, D), dtype=np.float32) * scales[None, :, None])
        k = wl.normal_bf16(rng, (T, hkv, D))
        v = wl.normal_bf16(rng, (T, hkv, D))
        o = pkv.attn_prefill_varlen(to_dev(q, dev), to_dev(k, dev), to_dev(v, dev), to_dev(cu, dev),
                                    to_dev(cu, dev), max(lens), max(lens))
        ref = oracle.attn_prefill(q, k, v, cu, cu, hq, hkv)
    torch.cuda.synchronize()
    got = f64(o)
    mx, mean = check_attn(got, ref, "prefill, larger scores")
    per_head = np.abs(got - ref).max(axis=(0, 2))
    _say(f"  max |err| {mx:.3e}, mean {mean:.3e}; per head (x3 .. x9): {per_head[0]:.2e} .. {per_head[-1]:.2e}")


def test_prefill_two_pass_batch_full_rows(dev):
    """8 x 1024 tokens at 16/8 heads (about 7e10 FLOP counted without the causal half, so
    the fast pass runs): every (token, head) row against the oracle."""
    _say("prefill 8 x 1024 at 16/8 heads (fast + exact pass), all rows")
    rng = wl.rng_for(136, 0, 0)
    lens, hq, hkv = [1024] * 8, 16, 8
    T = sum(lens)
    cu = wl.cu_seqlens(lens)
    q = wl.normal_bf16(rng, (T, hq, D))
    k = wl.normal_bf16(rng, (T, hkv, D))
    v = wl.normal_bf16(rng, (T, hkv, D))
    o = pkv.attn_prefill_varlen(to_dev(q, dev), to_dev(k, dev), to_dev(v, dev), to_dev(cu, dev), to_dev(cu, dev),
                                1024, 1024)
    torch.cuda.synchronize()
    mx, mean = check_attn(f64(o), oracle.attn_prefill(q, k, v, cu, cu, hq, hkv), "prefill 8 x 1024")
    _say(f"  max |err| {mx:.3e}, mean {mean:.3e}")


def test_single_rounding_against_the_pages_rounding_points(dev):
    """The kernel keeps QK-Norm + RoPE in fp32 and rounds once; the pages' code rounds to
    bf16 after normalising, after the product with gamma and after the rotation.  The
    two q'/k' differ by a few bf16 steps at most, and attention over either stays inside
    the attention gates of the oracle's (unrounded) result.  Reported, with the counts."""
    w = wl.tiny_chain(seed=0)
    s = w.shape
    q0, k0, v0 = wl.qkv_views(s)
    n = w.qkv.shape[0]
    table = pkv.rope_cache_build(40960, D, 1e6, device=dev)
    th = oracle.rope_table(40960, D, 1e6)
    qkv = to_dev(w.qkv, dev)
    qo, ko = pkv.qk_norm_rope(qkv[:, q0:k0].view(n, 16, D), qkv[:, k0:v0].view(n, 8, D), to_dev(w.positions, dev),
                              to_dev(w.gamma_q, dev), to_dev(w.gamma_k, dev), table, s.eps)
    torch.cuda.synchronize()
    gq, gk = f64(qo), f64(ko)
    pq = oracle.rmsnorm_rope(w.qkv, 16, D, w.gamma_q, s.eps, w.positions, th, col_offset=q0, pages_rounding=True)
    pk = oracle.rmsnorm_rope(w.qkv, 8, D, w.gamma_k, s.eps, w.positions, th, col_offset=k0, pages_rounding=True)
    exact_q = oracle.rmsnorm_rope(w.qkv, 16, D, w.gamma_q, s.eps, w.positions, th, col_offset=q0)
    diff_frac = float(np.mean(np.concatenate([(gq != pq).ravel(), (gk != pk).ravel()])))
    pair = np.sqrt(exact_q[..., :64] ** 2 + exact_q[..., 64:] ** 2)
    pair_step = np.exp2(np.floor(np.log2(np.maximum(np.concatenate([pair, pair], -1), 2.0 ** -126))) - 7)
    err_k = np.abs(gq - exact_q) / pair_step     # in bf16 steps of the rotated pair's length
    err_p = np.abs(pq - exact_q) / pair_step
    assert np.all(np.abs(gq - pq) <= 4 * pair_step), "single rounding and the pages' three differ by > 4 steps"
    vb = np.ascontiguousarray(w.qkv[:, v0:]).reshape(n, 8, D)
    ref = oracle.attn_prefill(oracle.round_bf16(exact_q), oracle.round_bf16(
        oracle.rmsnorm_rope(w.qkv, 8, D, w.gamma_k, s.eps, w.positions, th, col_offset=k0)), vb,
        w.cu_seqlens, w.cu_seqlens, 16, 8)
    o_pages = oracle.attn_prefill(oracle.round_bf16(pq), oracle.round_bf16(pk), vb, w.cu_seqlens, w.cu_seqlens, 16, 8)
    o_gpu = pkv.attn_prefill_varlen(qo, ko, qkv[:, v0:].view(n, 8, D), to_dev(w.cu_seqlens, dev),
                                    to_dev(w.cu_seqlens, dev), 300, 300)
    torch.cuda.synchronize()
    mx_g, mean_g = check_attn(f64(o_gpu), ref, "attention over the kernel's q', k'")
    mx_p, mean_p = check_attn(o_pages, ref, "attention over the pages-rounded q', k'")
    gap = np.abs(f64(o_gpu) - o_pages)
    _say(f"q'/k': {diff_frac:.4f} of values differ between single rounding and the pages' three; "
         f"|q'-exact| in bf16 steps of the pair length: kernel max {np.max(err_k):.2f} mean {np.mean(err_k):.3f}, "
         f"pages max {np.max(err_p):.2f} mean {np.mean(err_p):.3f}; attention vs oracle: kernel "
         f"{mx_g:.2e}/{mean_g:.2e}, pages pipeline {mx_p:.2e}/{mean_p:.2e}; kernel vs pages pipeline "
         f"{gap.max():.2e}/{gap.mean():.2e}")
