"""GPU parity of the fused QK-Norm + RoPE + cache scatter (pkv_qk_norm_rope_store).

Two claims are checked on the same seeded inputs:
  * against the oracle: q' and the cached k' rows within the QK-Norm/RoPE gate,
    value rows and every untouched cache byte bit-exact;
  * against the unfused HIP path (pkv_qk_norm_rope then pkv_store_kvcache):
    every output byte identical, since the fused kernel promises the same bits.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_gqa_amd as pkv
import workloads as wl
from gpu_helpers import bits, check_ulp, to_dev

pytestmark = pytest.mark.gpu
D = 128


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pkv.load_library()
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def table_dev(dev):
    return pkv.rope_cache_build(40960, D, 1e6, device=dev)


@pytest.fixture(scope="module")
def table_host():
    return oracle.rope_table(40960, D, 1e6)


def _say(*a):
    print("[gpu]", *a, flush=True)


def _fused_case(dev, table_dev, table_host, shape, qkv, gq, gk, pos, slots, num_blocks, seed, with_k_out=True):
    """Run fused and unfused paths on random-filled pools; check both claims."""
    q0, k0, v0 = wl.qkv_views(shape)
    n, hq, hkv = qkv.shape[0], shape.num_q_heads, shape.num_kv_heads
    rng = np.random.default_rng(seed)
    pool = rng.integers(0, 65536, size=(2, num_blocks, 256, hkv, D), dtype=np.uint16)
    qkv_d = to_dev(qkv, dev)
    q = qkv_d[:, q0:k0].view(n, hq, D)
    k = qkv_d[:, k0:v0].view(n, hkv, D)
    v = qkv_d[:, v0:].view(n, hkv, D)
    pos_d, slot_d = to_dev(pos.astype(np.int64), dev), to_dev(slots.astype(np.int32), dev)
    gq_d, gk_d = to_dev(gq, dev), to_dev(gk, dev)

    kc_f, vc_f = to_dev(pool[0], dev), to_dev(pool[1], dev)
    k_out = torch.empty((n, hkv, D), dtype=torch.bfloat16, device=dev) if with_k_out else None
    qo_f = pkv.qk_norm_rope_store(q, k, v, pos_d, gq_d, gk_d, table_dev, kc_f, vc_f, slot_d, shape.eps,
                                  k_out=k_out)
    kc_u, vc_u = to_dev(pool[0], dev), to_dev(pool[1], dev)
    qo_u, ko_u = pkv.qk_norm_rope(q, k, pos_d, gq_d, gk_d, table_dev, shape.eps)
    pkv.store_kvcache(ko_u, v, kc_u, vc_u, slot_d)
    torch.cuda.synchronize()

    # fused == unfused, byte for byte
    assert torch.equal(qo_f.view(torch.int16), qo_u.view(torch.int16)), "q' differs from the unfused path"
    assert torch.equal(kc_f.view(torch.int16), kc_u.view(torch.int16)), "k_cache differs from the unfused path"
    assert torch.equal(vc_f.view(torch.int16), vc_u.view(torch.int16)), "v_cache differs from the unfused path"
    if with_k_out:
        assert torch.equal(k_out.view(torch.int16), ko_u.view(torch.int16)), "k_out differs from the unfused path"

    # against the oracle
    ref_q = oracle.rmsnorm_rope(qkv, hq, D, gq, shape.eps, pos, table_host, col_offset=q0)
    ref_k = oracle.rmsnorm_rope(qkv, hkv, D, gk, shape.eps, pos, table_host, col_offset=k0)
    check_ulp(bits(qo_f).reshape(ref_q.shape), ref_q, oracle.round_bf16(ref_q), "q'")
    kc_got = bits(kc_f).reshape(-1, hkv, D)
    vc_got = bits(vc_f).reshape(-1, hkv, D)
    valid = (slots >= 0) & (slots < num_blocks * 256)
    vs = slots[valid]
    if valid.any():
        check_ulp(kc_got[vs], ref_k[valid], oracle.round_bf16(ref_k[valid]), "cached k'")
    # values and untouched bytes: the oracle's scatter of (cache k' as read back, v) over the same pool
    ek, ev = pool[0].reshape(-1, hkv, D).copy(), pool[1].reshape(-1, hkv, D).copy()
    vb = np.ascontiguousarray(qkv[:, v0:]).reshape(n, hkv, D)
    kb = np.zeros((n, hkv, D), np.uint16)
    kb[valid] = kc_got[vs]
    oracle.store_kvcache(kb, vb, ek, ev, slots.astype(np.int32))
    assert np.array_equal(kc_got, ek), "k_cache rows outside the written slots changed"
    assert np.array_equal(vc_got, ev), "v_cache differs from the oracle scatter"
    return qo_f


def test_fused_tiny_chain(dev, table_dev, table_host):
    _say("qk_norm_rope_store: tiny chain (337 tokens, 16/8 heads, one padding slot)")
    w = wl.tiny_chain(seed=0)
    slots = w.slot_mapping.copy()
    slots[5] = -1
    _fused_case(dev, table_dev, table_host, w.shape, w.qkv, w.gamma_q, w.gamma_k, w.positions, slots,
                w.num_blocks, seed=11)


def test_fused_8b_random_slots(dev, table_dev, table_host):
    _say("qk_norm_rope_store: 8B shapes, 777 tokens, -1 / out-of-range slots, no k_out")
    s = wl.QWEN3_8B
    rng = wl.rng_for(92, 0, 0)
    n, nb = 777, 8
    qkv = wl.normal_bf16(rng, (n, s.qkv_width), scale=3.0)
    gq, gk = wl.gamma_bf16(rng), wl.gamma_bf16(rng)
    pos = rng.integers(0, 40960, size=n).astype(np.int64)
    slots = rng.permutation(nb * 256)[:n].astype(np.int32)
    slots[:6] = [-1, nb * 256, -5, 0, nb * 256 - 1, -1]
    _fused_case(dev, table_dev, table_host, s, qkv, gq, gk, pos, slots, nb, seed=12, with_k_out=False)


def test_fused_8b_decode_batch(dev, table_dev, table_host):
    _say("qk_norm_rope_store: the 8B decode step (256 tokens at their cache slots)")
    w = wl.paged_decode_8b(seed=0)
    s = w.shape
    # the decode step's slots index a pool of w.num_blocks blocks; use a pool just large enough
    used = np.unique(w.slot_mapping // 256)
    remap = {int(b): i for i, b in enumerate(used)}
    slots = np.array([remap[int(x) // 256] * 256 + int(x) % 256 for x in w.slot_mapping], np.int32)
    _fused_case(dev, table_dev, table_host, s, w.qkv(), *w.gammas(), w.positions, slots, len(used), seed=13)


def test_fused_in_place_q(dev, table_dev, table_host):
    _say("qk_norm_rope_store: q_out aliasing a contiguous q")
    w = wl.tiny_chain(seed=1)
    s = w.shape
    q0, k0, v0 = wl.qkv_views(s)
    n = w.qkv.shape[0]
    qkv_d = to_dev(w.qkv, dev)
    q = qkv_d[:, q0:k0].contiguous().view(n, 16, D)
    k = qkv_d[:, k0:v0].contiguous().view(n, 8, D)
    v = qkv_d[:, v0:].view(n, 8, D)
    kc = torch.zeros((w.num_blocks, 256, 8, D), dtype=torch.bfloat16, device=dev)
    vc = torch.zeros_like(kc)
    pos, slot = to_dev(w.positions, dev), to_dev(w.slot_mapping, dev)
    gq, gk = to_dev(w.gamma_q, dev), to_dev(w.gamma_k, dev)
    ref_q = pkv.qk_norm_rope_store(q, k, v, pos, gq, gk, table_dev, kc.clone(), vc.clone(), slot, s.eps)
    pkv.qk_norm_rope_store(q, k, v, pos, gq, gk, table_dev, kc, vc, slot, s.eps, q_out=q, k_out=k)
    qo_u, ko_u = pkv.qk_norm_rope(qkv_d[:, q0:k0].view(n, 16, D), qkv_d[:, k0:v0].view(n, 8, D), pos, gq, gk,
                                  table_dev, s.eps)
    torch.cuda.synchronize()
    assert torch.equal(q.view(torch.int16), ref_q.view(torch.int16))
    assert torch.equal(q.view(torch.int16), qo_u.view(torch.int16))
    assert torch.equal(k.view(torch.int16), ko_u.view(torch.int16))


@pytest.mark.parametrize("hq,hkv,n", [(6, 2, 1), (6, 2, 5), (6, 2, 3000), (12, 4, 2500), (40, 8, 2049), (2, 1, 700)])
def test_fused_odd_head_counts_and_token_counts(dev, table_dev, table_host, hq, hkv, n):
    """Head counts that are not multiples of 4 and token counts on both sides of the
    point where the kernels stop splitting a token's heads over several waves."""
    _say(f"qk_norm_rope_store: {hq}/{hkv} heads, {n} tokens")
    s = wl.Shape(num_q_heads=hq, num_kv_heads=hkv)
    rng = wl.rng_for(95, hq * 1000 + n, 0)
    qkv = wl.normal_bf16(rng, (n, s.qkv_width), scale=2.0)
    gq, gk = wl.gamma_bf16(rng), wl.gamma_bf16(rng)
    pos = rng.integers(0, 40960, size=n).astype(np.int64)
    nb = (n + 255) // 256 + 1
    slots = rng.permutation(nb * 256)[:n].astype(np.int32)
    slots[0] = -1                    # a padding token
    if n > 2:
        slots[2] = nb * 256          # a slot past the pool: skipped like -1
    _fused_case(dev, table_dev, table_host, s, qkv, gq, gk, pos, slots, nb, seed=hq + n)


@pytest.mark.parametrize("case", range(8))
def test_fused_random_shapes(dev, table_dev, table_host, case):
    """Seeded random head counts (kv heads 1-8, groups 1-8), token counts (log-uniform up to
    4000), input scales, positions over the whole table and slot maps with padding."""
    rng = wl.rng_for(96, case, 0)
    hkv = int(rng.choice([1, 2, 4, 8]))
    hq = hkv * int(rng.integers(1, 9))
    n = int(np.exp(rng.uniform(0, np.log(4001))))
    s = wl.Shape(num_q_heads=hq, num_kv_heads=hkv)
    _say(f"qk_norm_rope_store random case {case}: {hq}/{hkv} heads, {n} tokens")
    qkv = wl.normal_bf16(rng, (n, s.qkv_width), scale=float(rng.choice([0.25, 2.0, 16.0])))
    gq, gk = wl.gamma_bf16(rng), wl.gamma_bf16(rng)
    pos = rng.integers(0, 40960, size=n).astype(np.int64)
    nb = (n + 255) // 256 + int(rng.integers(1, 4))
    slots = rng.permutation(nb * 256)[:n].astype(np.int32)
    slots[rng.random(n) < 0.05] = -1
    _fused_case(dev, table_dev, table_host, s, qkv, gq, gk, pos, slots, nb, seed=900 + case)
