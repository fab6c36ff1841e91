"""GPU parity on seeded random shapes.

Each case draws its own batch size, GQA group, kv heads, lengths (log-uniform, with
empty sequences), cached prefixes and block placement, so the launch paths (exact
pass alone or two passes, 4- or 8-wave workgroups, key split, dealing windows,
sub-block decode splits, size-ordered dispatch) meet shapes no hand-written case
picked.  Prefill: the first and last row of every sequence and 96 random rows
against the oracle; decode: every row against the oracle; decode step: byte-equal
to QK-Norm + RoPE + scatter followed by the decode call.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_gqa_amd as pkv
import workloads as wl
from gpu_helpers import check_attn, f64, to_dev

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


def _log_uniform(rng, lo, hi, n):
    return np.floor(np.exp(rng.uniform(np.log(lo), np.log(hi + 1), n))).astype(np.int64)


def _heads(rng):
    hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 4, 8] + ([16] if hkv <= 4 else [])))
    return hkv * g, hkv


def _paged_pool(rng, lens_k, hkv):
    """A permuted pool holding each sequence's keys; -1 padding in the table."""
    nb = sum(-(-int(L) // 256) for L in lens_k) + 3
    perm = rng.permutation(nb)
    rows_bt, nxt = [], 0
    for L in lens_k:
        c = -(-int(L) // 256)
        rows_bt.append(list(perm[nxt:nxt + c]))
        nxt += c
    return nb, wl.pad_block_tables(rows_bt, max(1, max(len(r) for r in rows_bt)))


@pytest.mark.parametrize("case", range(16))
def test_prefill_random_shapes(dev, case):
    rng = wl.rng_for(99, case, 0)
    hq, hkv = _heads(rng)
    B = int(rng.integers(1, 13))
    lens_q = _log_uniform(rng, 1, 3000, B)
    lens_q[rng.random(B) < 0.15] = 0
    paged = bool(rng.random() < 0.5)
    if lens_q.sum() == 0:
        lens_q[0] = 1
    lens_k = lens_q + (rng.integers(0, 3001, B) if paged else 0)
    _say(f"prefill random case {case}: {hq}/{hkv} heads, paged={paged}, Lq {lens_q.tolist()}, Lk {lens_k.tolist()}")
    cuq, cuk = wl.cu_seqlens(lens_q), wl.cu_seqlens(lens_k)
    tq, tk = int(cuq[-1]), int(cuk[-1])
    q = wl.normal_bf16(rng, (tq, hq, D))
    k = wl.normal_bf16(rng, (tk, hkv, D))
    v = wl.normal_bf16(rng, (tk, hkv, D))
    rows = [[int(cuq[b]), h] for b in range(B) if lens_q[b] for h in (0, hq - 1)]
    rows += [[int(cuq[b + 1]) - 1, h] for b in range(B) if lens_q[b] for h in (0, hq - 1)]
    rows += np.stack([rng.integers(0, tq, 96), rng.integers(0, hq, 96)], 1).tolist()
    rows = np.array(rows, np.int64)
    if not paged:
        o = pkv.attn_prefill_varlen(to_dev(q, dev), to_dev(k, dev), to_dev(v, dev), to_dev(cuq, dev), to_dev(cuk, dev),
                                    int(lens_q.max()), int(lens_k.max()))
        torch.cuda.synchronize()
        ref = oracle.attn_prefill(q, k, v, cuq, cuk, hq, hkv, rows=rows)
    else:
        nb, bt = _paged_pool(rng, lens_k, hkv)
        kc = wl.normal_bf16(rng, (nb * 256, hkv, D))
        vc = wl.normal_bf16(rng, (nb * 256, hkv, D))
        off = 0
        for b, L in enumerate(lens_k):
            sl = wl.slots_for(bt[b], np.arange(int(L)))
            kc[sl] = k[off:off + L]
            vc[sl] = v[off:off + L]
            off += int(L)
        o = pkv.attn_prefill_varlen(to_dev(q, dev), to_dev(kc.reshape(nb, 256, hkv, D), dev),
                                    to_dev(vc.reshape(nb, 256, hkv, D), dev), to_dev(cuq, dev), to_dev(cuk, dev),
                                    int(lens_q.max()), int(lens_k.max()), block_table=to_dev(bt, dev))
        torch.cuda.synchronize()
        ref = oracle.attn_prefill(q, kc, vc, cuq, cuk, hq, hkv, block_table=bt, rows=rows)
    check_attn(f64(o)[rows[:, 0], rows[:, 1]], ref, f"prefill random case {case}")


@pytest.mark.parametrize("case", range(16))
def test_decode_random_shapes(dev, case):
    rng = wl.rng_for(98, case, 0)
    hq, hkv = _heads(rng)
    B = int(rng.integers(1, 41))
    ctx = _log_uniform(rng, 1, 20000, B)
    ctx[rng.random(B) < 0.1] = 0
    _say(f"decode random case {case}: {hq}/{hkv} heads, batch {B}, contexts up to {int(ctx.max())}")
    nb, bt = _paged_pool(rng, np.maximum(ctx, 1), hkv)
    kc = wl.normal_bf16(rng, (nb, 256, hkv, D))
    vc = wl.normal_bf16(rng, (nb, 256, hkv, D))
    q = wl.normal_bf16(rng, (B, hq, D))
    cl = ctx.astype(np.int32)
    o = pkv.attn_decode_paged(to_dev(q, dev), to_dev(kc, dev), to_dev(vc, dev), to_dev(cl, dev), to_dev(bt, dev))
    torch.cuda.synchronize()
    got = f64(o)
    live = cl > 0
    if live.any():
        ref = oracle.attn_decode(q[live], kc.reshape(-1, hkv, D), vc.reshape(-1, hkv, D), cl[live], bt[live], hq, hkv)
        check_attn(got[live], ref, f"decode random case {case}")
    assert np.all(got[~live] == 0.0), "an empty context must give a zero row"


@pytest.mark.parametrize("case", range(6))
def test_decode_step_random_shapes(dev, case):
    rng = wl.rng_for(97, case, 1)
    hq, hkv = _heads(rng)
    B = int(rng.integers(1, 70))
    width = (hq + 2 * hkv) * D
    ctx = _log_uniform(rng, 1, 6000, B)
    _say(f"decode step random case {case}: {hq}/{hkv} heads, batch {B}, contexts up to {int(ctx.max())}")
    nb, bt = _paged_pool(rng, ctx, hkv)
    pos = ctx - 1
    slots = np.array([bt[i, pos[i] // 256] * 256 + pos[i] % 256 for i in range(B)], np.int32)
    qkv = wl.normal_bf16(rng, (B, width))
    pool = wl.normal_bf16(rng, (2, nb, 256, hkv, D))
    gq, gk = wl.gamma_bf16(rng), wl.gamma_bf16(rng)
    table = pkv.rope_cache_build(40960, D, 1e6, device=dev)
    gq_d, gk_d = to_dev(gq, dev), to_dev(gk, dev)
    qkv_d, pos_d, slot_d, ctx_d, bt_d = (to_dev(x, dev) for x in (qkv, pos, slots, ctx.astype(np.int32), bt))
    kc1, vc1 = to_dev(pool[0], dev), to_dev(pool[1], dev)
    st = pkv.DecodeStep(qkv_d, kc1, vc1, pos_d, slot_d, ctx_d, bt_d, gq_d, gk_d, table, hq, hkv, eps=1e-6)
    st.run(B)
    kc2, vc2 = to_dev(pool[0], dev), to_dev(pool[1], dev)
    q0, k0 = hq * D, (hq + hkv) * D
    q_out = pkv.qk_norm_rope_store(qkv_d[:, :q0].view(B, hq, D), qkv_d[:, q0:k0].view(B, hkv, D),
                                   qkv_d[:, k0:].view(B, hkv, D), pos_d, gq_d, gk_d, table, kc2, vc2, slot_d, eps=1e-6)
    o2 = pkv.attn_decode_paged(q_out, kc2, vc2, ctx_d, bt_d)
    torch.cuda.synchronize()
    assert torch.equal(st.q_out[:B].view(torch.int16), q_out.view(torch.int16)), "q'"
    assert torch.equal(kc1.view(torch.int16), kc2.view(torch.int16)), "k_cache"
    assert torch.equal(vc1.view(torch.int16), vc2.view(torch.int16)), "v_cache"
    assert torch.equal(st.o[:B].view(torch.int16), o2.view(torch.int16)), "o"
    st.close()
