"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Every input comes from the seeded generators in ``workloads``; every expected
value from ``oracle``.  Gates are in tests/gpu_helpers.py.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import paged_kv_gqa_amd as pkv
import workloads as wl
from gpu_helpers import (bits, check_attn, check_ulp, f64, gather_sequences, to_dev)

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


# ---------------------------------------------------------------------------
# RoPE table and QK-Norm + RoPE
# ---------------------------------------------------------------------------

def test_rope_table_matches_oracle(dev, table_dev, table_host):
    _say("rope table 40960 x 128")
    got = table_dev.cpu().numpy()
    ulps = np.abs(got.view(np.int32).astype(np.int64) - table_host.view(np.int32).astype(np.int64))
    assert ulps.max() <= 1, f"table differs by {ulps.max()} fp32 ulps"


def _norm_rope_case(dev, table_dev, table_host, shape, qkv, gq, gk, pos):
    q0, k0, _ = wl.qkv_views(shape)
    n = qkv.shape[0]
    qkv_d = to_dev(qkv, dev)
    q = qkv_d[:, q0:k0].view(n, shape.num_q_heads, D)
    k = qkv_d[:, k0:k0 + shape.kv_size].view(n, shape.num_kv_heads, D)
    pos_d = to_dev(pos.astype(np.int64), dev)
    qo, ko = pkv.qk_norm_rope(q, k, pos_d, to_dev(gq, dev), to_dev(gk, dev), table_dev, shape.eps)
    torch.cuda.synchronize()
    ref_q = oracle.rmsnorm_rope(qkv, shape.num_q_heads, D, gq, shape.eps, pos, table_host, col_offset=q0)
    ref_k = oracle.rmsnorm_rope(qkv, shape.num_kv_heads, D, gk, shape.eps, pos, table_host, col_offset=k0)
    check_ulp(bits(qo).reshape(ref_q.shape), ref_q, oracle.round_bf16(ref_q), "q'")
    check_ulp(bits(ko).reshape(ref_k.shape), ref_k, oracle.round_bf16(ref_k), "k'")
    return qkv_d, qo, ko


def test_qk_norm_rope_tiny(dev, table_dev, table_host):
    _say("qk_norm_rope on the two-sequence chain (337 tokens, 16/8 heads)")
    w = wl.tiny_chain(seed=0)
    qkv_d, qo, ko = _norm_rope_case(dev, table_dev, table_host, w.shape, w.qkv, w.gamma_q, w.gamma_k, w.positions)
    # in place on contiguous copies gives the same bits
    n = w.qkv.shape[0]
    qc = qkv_d[:, :2048].contiguous().view(n, 16, D)
    kc = qkv_d[:, 2048:3072].contiguous().view(n, 8, D)
    pkv.qk_norm_rope(qc, kc, to_dev(w.positions, dev), to_dev(w.gamma_q, dev), to_dev(w.gamma_k, dev), table_dev,
                     1e-6, q_out=qc, k_out=kc)
    torch.cuda.synchronize()
    assert torch.equal(qc, qo) and torch.equal(kc, ko)


def test_qk_norm_rope_8b_long_positions(dev, table_dev, table_host):
    _say("qk_norm_rope 8B shapes, 777 tokens, positions up to 40959")
    s = wl.QWEN3_8B
    rng = wl.rng_for(90, 0, 0)
    qkv = wl.normal_bf16(rng, (777, s.qkv_width), scale=3.0)
    gq, gk = wl.gamma_bf16(rng), wl.gamma_bf16(rng)
    pos = rng.integers(0, 40960, size=777).astype(np.int64)
    pos[:2] = [0, 40959]
    _norm_rope_case(dev, table_dev, table_host, s, qkv, gq, gk, pos)


# ---------------------------------------------------------------------------
# store_kvcache
# ---------------------------------------------------------------------------

def _store_raw(key, value, kc, vc, slots, hkv, hd, key_stride=None, value_stride=None):
    lib = pkv.load_library()
    rc = lib.pkv_store_kvcache(key.data_ptr(), key_stride or hkv * hd, value.data_ptr(), value_stride or hkv * hd,
                               kc.data_ptr(), vc.data_ptr(), kc.numel() // (hkv * hd), slots.data_ptr(),
                               slots.numel(), hkv, hd, key.element_size(),
                               torch.cuda.current_stream().cuda_stream)
    assert rc == 0, lib.pkv_last_error()


def test_store_kvcache_printed_examples(dev, golden):
    _say("store_kvcache printed examples (fp32 rows)")
    g = golden("scatter_skeleton_w3.json")
    src = torch.tensor(g["src"], dtype=torch.float32, device=dev)
    dk, dv = torch.zeros(3, 4, device=dev), torch.zeros(3, 4, device=dev)
    _store_raw(src, src, dk, dv, torch.tensor(g["slot"], dtype=torch.int32, device=dev), 1, 4)
    torch.cuda.synchronize()
    assert dk.cpu().tolist() == g["expected_dst"]
    g = golden("store_kvcache_w4.json")
    base = torch.arange(4).reshape(1, 2, 2)
    key = (torch.arange(4).reshape(4, 1, 1) * 10 + base).float().to(dev)
    value = key + 100
    kc = torch.zeros(g["cache_shape"], device=dev)
    vc = torch.zeros(g["cache_shape"], device=dev)
    _store_raw(key, value, kc, vc, torch.tensor(g["slot_mapping"], dtype=torch.int32, device=dev), 2, 2)
    torch.cuda.synchronize()
    assert kc.view(-1, 4).cpu().tolist() == g["expected_k_cache_rows"]
    assert vc.view(-1, 4)[0].cpu().tolist() == g["expected_v_cache_slot0"]


def _store_vs_oracle(dev, key_np, val_np, slots, num_blocks, hkv, key_stride, val_stride, seed):
    """Random bytes in the caches first: every byte the scatter must not touch is checked too."""
    rng = np.random.default_rng(seed)
    kc0 = rng.integers(0, 65536, size=(num_blocks, 256, hkv, D), dtype=np.uint16)
    vc0 = rng.integers(0, 65536, size=(num_blocks, 256, hkv, D), dtype=np.uint16)
    kc, vc = to_dev(kc0, dev), to_dev(vc0, dev)
    kd, vd = to_dev(key_np, dev), to_dev(val_np, dev)
    n = slots.shape[0]
    key_v = torch.as_strided(kd, (n, hkv, D), (key_stride, D, 1))
    val_v = torch.as_strided(vd, (n, hkv, D), (val_stride, D, 1), storage_offset=0)
    pkv.store_kvcache(key_v, val_v, kc, vc, to_dev(slots, dev))
    torch.cuda.synchronize()
    ek, ev = kc0.copy(), vc0.copy()
    oracle.store_kvcache(key_np, val_np, ek, ev, slots, key_row_stride=key_stride, value_row_stride=val_stride,
                         row_elems=hkv * D)
    assert np.array_equal(bits(kc).reshape(ek.shape), ek)
    assert np.array_equal(bits(vc).reshape(ev.shape), ev)


def test_store_kvcache_bit_exact_tiny_chain(dev):
    _say("store_kvcache tiny chain, v as a strided view of qkv")
    w = wl.tiny_chain(seed=0)
    n = w.qkv.shape[0]
    key = np.ascontiguousarray(w.qkv[:, 2048:3072])          # contiguous k rows
    val = np.ascontiguousarray(w.qkv[:, 3072:])              # v columns of qkv: row stride 4096 below
    qkv_v = np.zeros((n, 4096), np.uint16)
    qkv_v[:, :1024] = val
    slots = w.slot_mapping.copy()
    slots[5] = -1                                             # one padding token
    _store_vs_oracle(dev, key, qkv_v, slots, w.num_blocks, 8, 1024, 4096, seed=1)


def test_store_kvcache_bit_exact_8b_prefill(dev):
    _say("store_kvcache 32768 tokens (8B prefix workload)")
    w = wl.prefix_prefill_8b(seed=0)
    rng = wl.rng_for(91, 0, 0)
    key = rng.integers(0, 65536, size=(w.num_q_tokens, 1024), dtype=np.uint16)
    val = rng.integers(0, 65536, size=(w.num_q_tokens, 1024), dtype=np.uint16)
    _store_vs_oracle(dev, key, val, w.slot_mapping, w.num_blocks, 8, 1024, 1024, seed=2)


def test_store_kvcache_skips_out_of_range_slots(dev):
    _say("store_kvcache with -1 and out-of-range slots")
    rng = np.random.default_rng(3)
    key = rng.integers(0, 65536, size=(6, 1024), dtype=np.uint16)
    slots = np.array([0, -1, 511, 512, -7, 3], np.int32)     # pool of 2 blocks = 512 slots
    _store_vs_oracle(dev, key, key.copy(), slots, 2, 8, 1024, 1024, seed=4)


# ---------------------------------------------------------------------------
# prefill
# ---------------------------------------------------------------------------

def _prefill_case(dev, lens_q, lens_k, hq, hkv, seed, paged=False, num_blocks=None, rows=None, make_qkv=None):
    rng = wl.rng_for(92, seed, 0)
    cuq, cuk = wl.cu_seqlens(lens_q), wl.cu_seqlens(lens_k)
    tq, tk = int(cuq[-1]), int(cuk[-1])
    if make_qkv is None:
        q = wl.normal_bf16(rng, (tq, hq, D))
        k = wl.normal_bf16(rng, (tk, hkv, D))
        v = wl.normal_bf16(rng, (tk, hkv, D))
    else:
        q, k, v = make_qkv(rng, tq, tk)
    if not paged:
        o = pkv.attn_prefill_varlen(to_dev(q, dev), to_dev(k, dev), to_dev(v, dev), to_dev(cuq, dev),
                                    to_dev(cuk, dev), max(lens_q), max(lens_k))
        torch.cuda.synchronize()
        ref = oracle.attn_prefill(q, k, v, cuq, cuk, hq, hkv, rows=rows)
        return o, ref, (q, k, v, cuq, cuk)
    nb = num_blocks or sum(-(-L // 256) for L in lens_k) + 3
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
    o = pkv.attn_prefill_varlen(to_dev(q, dev), to_dev(kc.reshape(nb, 256, hkv, D), dev),
                                to_dev(vc.reshape(nb, 256, hkv, D), dev), to_dev(cuq, dev), to_dev(cuk, dev),
                                max(lens_q), max(lens_k), block_table=to_dev(bt, dev))
    torch.cuda.synchronize()
    ref = oracle.attn_prefill(q, kc, vc, cuq, cuk, hq, hkv, block_table=bt, rows=rows)
    return o, ref, (q, kc, vc, cuq, cuk, bt)


@pytest.mark.parametrize("hq,hkv", [(16, 8), (32, 8), (8, 8), (64, 8), (4, 2)])
def test_prefill_varlen_ragged(dev, hq, hkv):
    lens = [1, 37, 63, 64, 65, 129, 300]
    _say(f"prefill case 1, lengths {lens}, {hq}/{hkv} heads")
    o, ref, _ = _prefill_case(dev, lens, lens, hq, hkv, seed=hq + hkv)
    check_attn(f64(o), ref, "prefill ragged")


@pytest.mark.parametrize("lens_q,lens_k,paged", [
    ([0, 1500, 0, 1200, 7, 0], [0, 1500, 0, 1200, 7, 0], False),      # case 1: empty sequences between others
    ([0, 700, 0, 900, 0], [512, 1400, 300, 900, 0], True),            # case 2: cached keys but no new queries
])
def test_prefill_zero_length_sequences(dev, lens_q, lens_k, paged):
    """Sequences with no queries inside a batch produce no rows and leave the other
    sequences' rows as the oracle computes them.  32/8 heads and these sizes take the
    two-launch path (fast pass, then the exact pass), so both kernels meet the empty entries."""
    _say(f"prefill with zero-length sequences: q {lens_q}, k {lens_k}, paged={paged}")
    o, ref, _ = _prefill_case(dev, lens_q, lens_k, 32, 8, seed=41 + paged, paged=paged)
    assert o.shape[0] == sum(lens_q)
    check_attn(f64(o), ref, "prefill with empty sequences")


@pytest.mark.parametrize("lens,paged", [
    ([700, 150, 333], False),                  # exact pass alone; 22 query blocks per unit (rounds of 4 and a tail of 2)
    ([1500, 400, 1100], False),                # fast + exact pass; 47 blocks per unit (tail of 3)
    ([90, 1800, 5, 640, 1210, 0, 333], True),  # seven units per XCD, one sequence empty, over the paged cache
])
def test_prefill_small_ragged_batches_dealt_in_windows(dev, lens, paged):
    """Small ragged batches (at most 8 units per XCD, little K/V) deal each XCD's units
    together, heaviest query blocks of all of them first, in rounds of 4 blocks per unit.
    Every row of every sequence is still computed once: all rows against the oracle."""
    _say(f"prefill small ragged batch in dealing windows: lengths {lens}, paged={paged}")
    lens_k = [l + 64 * i for i, l in enumerate(lens)] if paged else lens
    o, ref, _ = _prefill_case(dev, lens, lens_k, 32, 8, seed=59 + len(lens), paged=paged)
    assert o.shape[0] == sum(lens)
    check_attn(f64(o), ref, "prefill in dealing windows")


def test_cache_offsets_past_2_31_elements(dev):
    """A 9000-block pool (4.7 GB per cache at 8 kv heads): blocks past 8192 start beyond
    2^31 elements, so every cache address must be formed in 64 bits.  The same contents
    placed at the end of the large pool give byte-identical prefill output, and both
    scatters write the same bytes there as the oracle / a compact pool."""
    hq, hkv, nb_big = 32, 8, 9000
    _say(f"cache offsets past 2^31 elements: {nb_big}-block pool, prefill case 2 and both scatters")
    lens_q, lens_k = [600, 300], [1500, 900]
    o_small, ref, (q, kc, vc, cuq, cuk, bt) = _prefill_case(dev, lens_q, lens_k, hq, hkv, seed=77, paged=True)
    nb_small = kc.shape[0] // 256
    base = nb_big - nb_small - 24                      # > 8192: element offsets past 2^31
    big_k = torch.empty((nb_big, 256, hkv, D), dtype=torch.bfloat16, device=dev)
    big_v = torch.empty_like(big_k)
    big_k[base:base + nb_small] = to_dev(kc.reshape(nb_small, 256, hkv, D), dev)
    big_v[base:base + nb_small] = to_dev(vc.reshape(nb_small, 256, hkv, D), dev)
    bt_big = np.where(bt >= 0, bt + base, -1).astype(np.int32)
    o_big = pkv.attn_prefill_varlen(to_dev(q, dev), big_k, big_v, to_dev(cuq, dev), to_dev(cuk, dev),
                                    max(lens_q), max(lens_k), block_table=to_dev(bt_big, dev))
    torch.cuda.synchronize()
    assert torch.equal(o_big.view(torch.int16), o_small.view(torch.int16)), "output depends on where the blocks sit"
    check_attn(f64(o_big), ref, "prefill, blocks past 2^31 elements")

    # scatter: 300 tokens into the last 10 blocks (zeroed first), against the oracle scatter
    rng = wl.rng_for(93, 3, 0)
    n, tail = 300, 10
    key, val = wl.normal_bf16(rng, (n, hkv, D)), wl.normal_bf16(rng, (n, hkv, D))
    local = rng.permutation(tail * 256)[:n].astype(np.int32)
    local[:3] = [-1 - (nb_big - tail) * 256, 0, tail * 256 - 1]   # first maps to slot -1
    slots = (local + (nb_big - tail) * 256).astype(np.int32)
    big_k[nb_big - tail:].zero_()
    big_v[nb_big - tail:].zero_()
    pkv.store_kvcache(to_dev(key, dev), to_dev(val, dev), big_k, big_v, to_dev(slots, dev))
    ek = np.zeros((tail * 256, hkv, D), np.uint16)
    ev = np.zeros_like(ek)
    oracle.store_kvcache(key, val, ek, ev, np.where(slots >= 0, local, -1).astype(np.int32))
    torch.cuda.synchronize()
    assert np.array_equal(bits(big_k[nb_big - tail:]).reshape(ek.shape), ek)
    assert np.array_equal(bits(big_v[nb_big - tail:]).reshape(ev.shape), ev)

    # fused QK-Norm + RoPE + scatter: the same bytes as into a compact pool of `tail` blocks
    qkv = wl.normal_bf16(rng, (n, (hq + 2 * hkv) * D))
    q0, k0, v0 = hq * D, (hq + hkv) * D, (hq + 2 * hkv) * D
    qkv_d = to_dev(qkv, dev)
    qv, kv, vv = (qkv_d[:, :q0].view(n, hq, D), qkv_d[:, q0:k0].view(n, hkv, D), qkv_d[:, k0:v0].view(n, hkv, D))
    pos = to_dev(rng.integers(0, 40960, size=n).astype(np.int64), dev)
    g = to_dev(wl.gamma_bf16(rng), dev)
    table = pkv.rope_cache_build(40960, D, 1e6, device=dev)
    big_k[nb_big - tail:].zero_()
    big_v[nb_big - tail:].zero_()
    qa = pkv.qk_norm_rope_store(qv, kv, vv, pos, g, g, table, big_k, big_v, to_dev(slots, dev), 1e-6)
    ck = torch.zeros((tail, 256, hkv, D), dtype=torch.bfloat16, device=dev)
    cv = torch.zeros_like(ck)
    qb = pkv.qk_norm_rope_store(qv, kv, vv, pos, g, g, table, ck, cv,
                                to_dev(np.where(slots >= 0, local, -1).astype(np.int32), dev), 1e-6)
    torch.cuda.synchronize()
    assert torch.equal(qa.view(torch.int16), qb.view(torch.int16))
    assert torch.equal(big_k[nb_big - tail:].view(torch.int16), ck.view(torch.int16))
    assert torch.equal(big_v[nb_big - tail:].view(torch.int16), cv.view(torch.int16))
    del big_k, big_v


def test_empty_calls_through_the_binding(dev):
    """Zero tokens / zero sequences: every entry point of the attention core returns
    without error, returns empty outputs and leaves the caches untouched."""
    _say("empty calls: qk_norm_rope, qk_norm_rope_store, store_kvcache, prefill, decode")
    hq, hkv = 16, 8
    bf = dict(dtype=torch.bfloat16, device=dev)
    q, k, v = torch.empty((0, hq, D), **bf), torch.empty((0, hkv, D), **bf), torch.empty((0, hkv, D), **bf)
    pos = torch.empty((0,), dtype=torch.int64, device=dev)
    slots = torch.empty((0,), dtype=torch.int32, device=dev)
    g = torch.ones((D,), **bf)
    table = pkv.rope_cache_build(4096, D, 1e6, device=dev)
    kc = torch.randn((2, 256, hkv, D), device=dev).to(torch.bfloat16)
    vc = torch.randn((2, 256, hkv, D), device=dev).to(torch.bfloat16)
    kc0, vc0 = kc.clone(), vc.clone()
    qo, ko = pkv.qk_norm_rope(q, k, pos, g, g, table, 1e-6)
    assert qo.shape == (0, hq, D) and ko.shape == (0, hkv, D)
    qo = pkv.qk_norm_rope_store(q, k, v, pos, g, g, table, kc, vc, slots, 1e-6)
    assert qo.shape == (0, hq, D)
    pkv.store_kvcache(k, v, kc, vc, slots)
    cu = torch.zeros((1,), dtype=torch.int32, device=dev)
    o = pkv.attn_prefill_varlen(q, k, v, cu, cu, 0, 0)
    assert o.shape == (0, hq, D)
    cu3 = torch.zeros((4,), dtype=torch.int32, device=dev)            # three sequences, all empty
    o = pkv.attn_prefill_varlen(q, kc, vc, cu3, cu3, 0, 0,
                                block_table=torch.full((3, 2), -1, dtype=torch.int32, device=dev))
    assert o.shape == (0, hq, D)
    od = pkv.attn_decode_paged(q, kc, vc, torch.empty((0,), dtype=torch.int32, device=dev),
                               torch.empty((0, 2), dtype=torch.int32, device=dev))
    assert od.shape == (0, hq, D)
    torch.cuda.synchronize()
    assert torch.equal(kc.view(torch.int16), kc0.view(torch.int16))
    assert torch.equal(vc.view(torch.int16), vc0.view(torch.int16))


@pytest.mark.parametrize("lens,hq,hkv", [([2100, 2500, 2048, 2300], 16, 8), ([2200, 3100], 32, 8), ([2048] * 3, 8, 4),
                                         ([2100, 2300], 64, 8), ([2048], 8, 8)])
def test_prefill_long_sequences_wide_workgroups(dev, lens, hq, hkv):
    """Mean query length >= 2048: 8-wave workgroups with 128-key tiles for every GQA group size."""
    _say(f"prefill case 1, lengths {lens}, {hq}/{hkv} heads (8-wave workgroups)")
    rows = np.stack([np.arange(0, sum(lens), 7), np.arange(0, sum(lens), 7) % hq], 1)
    o, ref, _ = _prefill_case(dev, lens, lens, hq, hkv, seed=len(lens) + hq, rows=rows)
    check_attn(f64(o)[rows[:, 0], rows[:, 1]], ref, "prefill long, 8 waves")
    lq = [L - 37 for L in lens] if sum(lens) - 37 * len(lens) >= 2048 * len(lens) else list(lens)
    rows = np.stack([np.arange(0, sum(lq), 5), np.arange(0, sum(lq), 5) % hq], 1)
    o2, ref2, _ = _prefill_case(dev, lq, lens, hq, hkv, seed=len(lens), paged=True, rows=rows)
    check_attn(f64(o2)[rows[:, 0], rows[:, 1]], ref2, "prefill long paged, 8 waves")


@pytest.mark.parametrize("lq,lk,hq,hkv", [([1024, 1300, 1111], [3000, 2700, 5000], 32, 8),
                                           ([1024, 1024], [2048, 2048], 64, 8),
                                           ([1500, 800, 1100], [4000, 900, 3100], 8, 2)])
def test_prefill_prefix_hits_medium_queries_wide_workgroups(dev, lq, lk, hq, hkv):
    """Four q heads a workgroup, 1024+ query positions on average and cached prefixes
    (longest key range at least twice the longest query): 8-wave workgroups."""
    assert sum(lq) >= 1024 * len(lq) and max(lk) >= 2 * max(lq) and hq // hkv >= 4
    _say(f"prefill case 2, queries {lq} over keys {lk}, {hq}/{hkv} heads (8-wave workgroups, prefix hits)")
    rows = np.stack([np.arange(0, sum(lq), 5), np.arange(0, sum(lq), 5) % hq], 1)
    o, ref, _ = _prefill_case(dev, lq, lk, hq, hkv, seed=sum(lq) + hq, paged=True, rows=rows)
    check_attn(f64(o)[rows[:, 0], rows[:, 1]], ref, "prefill prefix hits, 8 waves")


@pytest.mark.parametrize("lens,hq,hkv", [([1500], 4, 1), ([700, 90, 333], 4, 2), ([257], 8, 1)])
def test_prefill_few_work_units(dev, lens, hq, hkv):
    """Fewer (sequence, kv head) units than XCDs: the work is dealt in 2-block chunks."""
    _say(f"prefill case 1, lengths {lens}, {hq}/{hkv} heads (fewer than 8 units)")
    o, ref, _ = _prefill_case(dev, lens, lens, hq, hkv, seed=sum(lens) + hq)
    check_attn(f64(o), ref, "prefill few units")
    o2, ref2, _ = _prefill_case(dev, [min(64, L) for L in lens], lens, hq, hkv, seed=sum(lens), paged=True)
    check_attn(f64(o2), ref2, "prefill few units, paged")


def _extreme_scores(hq, hkv, kind):
    """q, k, v makers whose scores leave the range of the kernel's fast pass for a few
    query heads: 'large' scales those q rows by 40 (scores of several hundred in
    base-2 units, weights past 2^64 against a zero reference); 'small' points those
    q rows against a direction every key of kv head 0 shares (every score near -100
    in base-2 units, weights below 2^-64).  Other heads keep ordinary scores, so
    workgroups mixing both kinds of rows are exercised too."""
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
@pytest.mark.parametrize("lens_q,lens_k,hq,hkv,paged,step", [
    ([300, 700, 45], [300, 700, 45], 16, 8, False, 3),                  # exact pass alone, 4 waves
    ([2048], [2100], 4, 1, True, 3),                                    # exact pass alone, 8 waves
    ([4096, 4096], [4096, 4096], 32, 8, False, 7),                      # two passes, 8 waves, G = 4
    ([1024] * 40, [1024] * 40, 16, 8, False, 29),                       # two passes, 4 waves, G = 2
    ([1000] * 8, [8000] * 8, 8, 8, True, 7),                            # two passes, 4 waves, G = 1, paged
    ([1024] * 32, [1024] * 32, 32, 8, False, 23)])                      # two passes, 8192 work items
def test_prefill_scores_outside_fast_range(dev, kind, lens_q, lens_k, hq, hkv, paged, step):
    """Rows whose softmax sum leaves [2^-64, 2^64] against a zero reference are
    recomputed with the running-max pass; results match the oracle either way.
    The first two batches are small enough to run the exact pass alone (one
    launch); the others run both passes, with GQA groups of 4, 2 and 1, and (last
    case) far more work items than the exact pass has workgroups, so each of its
    workgroups walks several items."""
    _say(f"prefill, {kind} scores on some heads, Lq {lens_q[:3]}.. Lk {lens_k[:3]}.. ({len(lens_q)} seqs), "
         f"{hq}/{hkv} heads, paged={paged}")
    T = sum(lens_q)
    t = np.arange(0, T, step)
    rows = np.concatenate([np.stack([t, np.zeros_like(t)], 1), np.stack([t, np.full_like(t, hq - 1)], 1),
                           np.stack([t, (t // step) % hq], 1)])
    o, ref, _ = _prefill_case(dev, lens_q, lens_k, hq, hkv, seed=7 + hq, paged=paged, rows=rows,
                              make_qkv=_extreme_scores(hq, hkv, kind))
    got = f64(o)[rows[:, 0], rows[:, 1]]
    assert np.isfinite(got).all()
    check_attn(got, ref, f"prefill {kind} scores")


def test_prefill_flagged_and_clean_calls_on_two_streams(dev):
    """Two-pass prefill calls in flight together on two streams, one with rows that
    leave the fast pass's range and one without: each call's exact pass must find
    its own flags (the device keeps the highest flagged call number), whatever
    order the calls run in; the clean call may scan but stays exact."""
    _say("prefill: flagged and clean two-pass calls interleaved on two streams")
    hq, hkv = 32, 8
    lens_a, lens_b = [4096, 4096], [2048] * 4
    rng = wl.rng_for(92, 77, 0)
    qa, ka, va = _extreme_scores(hq, hkv, "large")(rng, sum(lens_a), sum(lens_a))
    qb = wl.normal_bf16(rng, (sum(lens_b), hq, D))
    kb = wl.normal_bf16(rng, (sum(lens_b), hkv, D))
    vb = wl.normal_bf16(rng, (sum(lens_b), hkv, D))
    cua, cub = wl.cu_seqlens(lens_a), wl.cu_seqlens(lens_b)
    da = [to_dev(x, dev) for x in (qa, ka, va, cua)]
    db = [to_dev(x, dev) for x in (qb, kb, vb, cub)]
    oa = torch.empty_like(da[0])
    ob = torch.empty_like(db[0])
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    for first in ("a", "b", "a"):
        oa.fill_(0)
        ob.fill_(0)
        torch.cuda.synchronize()
        order = [("a", s1), ("b", s2)] if first == "a" else [("b", s2), ("a", s1)]
        for which, st in order:
            with torch.cuda.stream(st):
                if which == "a":
                    pkv.attn_prefill_varlen(da[0], da[1], da[2], da[3], da[3], 4096, 4096, out=oa)
                else:
                    pkv.attn_prefill_varlen(db[0], db[1], db[2], db[3], db[3], 2048, 2048, out=ob)
        torch.cuda.synchronize()
        for q, k, v, cu, o, lens in ((qa, ka, va, cua, oa, lens_a), (qb, kb, vb, cub, ob, lens_b)):
            t = np.arange(0, sum(lens), 41)
            rows = np.concatenate([np.stack([t, np.zeros_like(t)], 1), np.stack([t, np.full_like(t, hq - 1)], 1)])
            ref = oracle.attn_prefill(q, k, v, cu, cu, hq, hkv, rows=rows)
            got = f64(o)[rows[:, 0], rows[:, 1]]
            assert np.isfinite(got).all()
            check_attn(got, ref, f"two streams, {first} first")


def test_prefill_captured_in_a_graph(dev):
    """Two-pass prefill calls captured into HIP graphs (one whose fast pass flags rows,
    one clean) and replayed several times, with eager prefill calls and other work
    between the replays: every replay gives the eager result byte for byte."""
    _say("prefill: two-pass calls captured into graphs and replayed")
    hq, hkv = 32, 8
    lens_a, lens_b = [4096, 4096], [2048] * 4
    rng = wl.rng_for(92, 78, 0)
    qa, ka, va = _extreme_scores(hq, hkv, "large")(rng, sum(lens_a), sum(lens_a))
    qb = wl.normal_bf16(rng, (sum(lens_b), hq, D))
    kb = wl.normal_bf16(rng, (sum(lens_b), hkv, D))
    vb = wl.normal_bf16(rng, (sum(lens_b), hkv, D))
    cua, cub = wl.cu_seqlens(lens_a), wl.cu_seqlens(lens_b)
    da = [to_dev(x, dev) for x in (qa, ka, va, cua)]
    db = [to_dev(x, dev) for x in (qb, kb, vb, cub)]
    ga, gb = torch.empty_like(da[0]), torch.empty_like(db[0])    # the graphs' outputs
    ea = pkv.attn_prefill_varlen(da[0], da[1], da[2], da[3], da[3], 4096, 4096)
    eb = pkv.attn_prefill_varlen(db[0], db[1], db[2], db[3], db[3], 2048, 2048)
    torch.cuda.synchronize()
    graphs = []
    for d, o, L in ((da, ga, 4096), (db, gb, 2048)):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):       # the binding enqueues on the capturing stream
            pkv.attn_prefill_varlen(d[0], d[1], d[2], d[3], d[3], L, L, out=o)
        graphs.append(g)
    torch.cuda.synchronize()
    for rep in range(3):
        ga.fill_(0)
        gb.fill_(0)
        order = graphs if rep % 2 == 0 else graphs[::-1]
        for g in order:
            g.replay()
        # eager work between replays: another flagged call and unrelated kernels
        extra = pkv.attn_prefill_varlen(da[0], da[1], da[2], da[3], da[3], 4096, 4096)
        junk = torch.randn(1 << 20, device=dev).sum()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        assert torch.equal(ga.view(torch.int16), ea.view(torch.int16)), f"replay {rep}: flagged call"
        assert torch.equal(gb.view(torch.int16), eb.view(torch.int16)), f"replay {rep}: clean call"
        assert torch.equal(extra.view(torch.int16), ea.view(torch.int16)), f"replay {rep}: eager call"
    t = np.arange(0, sum(lens_a), 37)
    rows = np.concatenate([np.stack([t, np.zeros_like(t)], 1), np.stack([t, np.full_like(t, hq - 1)], 1)])
    ref = oracle.attn_prefill(qa, ka, va, cua, cua, hq, hkv, rows=rows)
    check_attn(f64(ga)[rows[:, 0], rows[:, 1]], ref, "graph replay, flagged call")


def test_prefill_paged_prefix(dev):
    lk, lq = [300, 513, 64, 1000], [40, 257, 64, 1]
    _say(f"prefill case 2 (paged), Lk {lk}, Lq {lq}")
    o, ref, _ = _prefill_case(dev, lq, lk, 32, 8, seed=5, paged=True)
    check_attn(f64(o), ref, "prefill paged")


def test_prefill_paged_equals_contiguous(dev):
    lens = [100, 257, 512, 700]
    _say("prefill: paged and contiguous loaders give the same bits")
    o1, _, inp = _prefill_case(dev, lens, lens, 16, 8, seed=6)
    q, k, v, cuq, cuk = inp
    nb = sum(-(-L // 256) for L in lens) + 2
    perm = np.random.default_rng(7).permutation(nb)
    kc = np.zeros((nb * 256, 8, D), np.uint16)
    vc = np.zeros_like(kc)
    rows_bt, nxt, off = [], 0, 0
    for L in lens:
        c = -(-L // 256)
        rows_bt.append(list(perm[nxt:nxt + c]))
        nxt += c
    bt = wl.pad_block_tables(rows_bt)
    for b, L in enumerate(lens):
        sl = wl.slots_for(bt[b], np.arange(L))
        kc[sl], vc[sl] = k[off:off + L], v[off:off + L]
        off += L
    o2 = pkv.attn_prefill_varlen(to_dev(q, dev), to_dev(kc.reshape(nb, 256, 8, D), dev),
                                 to_dev(vc.reshape(nb, 256, 8, D), dev), to_dev(cuq, dev), to_dev(cuk, dev),
                                 max(lens), max(lens), block_table=to_dev(bt, dev))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_prefill_varlen_workload_full(dev):
    """The 0.6B varlen batch (8 sequences, lengths U[128, 2048], q/k/v as strided views
    of the qkv rows): every (token, head) row against the oracle."""
    w = wl.varlen_prefill(seed=0)
    s = w.shape
    _say(f"prefill 0.6B varlen workload, lengths {list(w.lengths)}, all rows")
    qkv = w.qkv()
    n = qkv.shape[0]
    q0, k0, v0 = wl.qkv_views(s)
    qkv_d = to_dev(qkv, dev)
    q = qkv_d[:, q0:k0].view(n, 16, D)
    k = qkv_d[:, k0:v0].view(n, 8, D)
    v = qkv_d[:, v0:].view(n, 8, D)
    cu = to_dev(w.cu_seqlens, dev)
    L = int(w.lengths.max())
    o = pkv.attn_prefill_varlen(q, k, v, cu, cu, L, L)
    torch.cuda.synchronize()
    ref = oracle.attn_prefill(qkv, qkv, qkv, w.cu_seqlens, w.cu_seqlens, 16, 8, q_row_stride=4096,
                              k_row_stride=4096, v_row_stride=4096, q_col=q0, k_col=k0, v_col=v0)
    mx, mean = check_attn(f64(o), ref, "prefill 0.6B varlen")
    _say(f"  max |err| {mx:.3e}, mean {mean:.3e} over {ref.shape[0] * ref.shape[1]} rows")


def test_prefill_prefix_workload_full(dev):
    """The 8B prefix-hit batch (16 x 2048 queries over 4096 paged keys, one shared 2048-token
    prefix), in the launch configuration the benchmark times: all 1,048,576 (token, head)
    rows against the oracle (about 1.65 TFLOP of fp64 loops on the host)."""
    w = wl.prefix_prefill_8b(seed=0)
    _say("prefill 8B prefix-hit workload (16 x 2048 queries over 4096 keys), all rows")
    rng = wl.rng_for(93, 0, 0)
    hkv, hq = 8, 32
    kc = torch.empty((w.num_blocks, 256, hkv, D), dtype=torch.bfloat16, device=dev)
    vc = torch.empty_like(kc)
    wl.fill_normal_bf16_(kc, 5, 0, 10)
    wl.fill_normal_bf16_(vc, 5, 0, 11)
    q = to_dev(wl.normal_bf16(rng, (w.num_q_tokens, hq, D)), dev)
    o = pkv.attn_prefill_varlen(q, kc, vc, to_dev(w.cu_seqlens_q, dev), to_dev(w.cu_seqlens_k, dev), 2048, 4096,
                                block_table=to_dev(w.block_tables, dev))
    torch.cuda.synchronize()
    ref = oracle.attn_prefill(bits(q), bits(kc).reshape(-1, hkv, D), bits(vc).reshape(-1, hkv, D), w.cu_seqlens_q,
                              w.cu_seqlens_k, hq, hkv, block_table=w.block_tables)
    mx, mean = check_attn(f64(o), ref, "prefill 8B prefix")
    _say(f"  max |err| {mx:.3e}, mean {mean:.3e} over {ref.shape[0] * ref.shape[1]} rows")


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------

def _decode_case(dev, ctx, hq, hkv, seed, nan_canaries=False, permute=False):
    rng = wl.rng_for(94, seed, 0)
    B = len(ctx)
    mb = max(-(-c // 256) for c in ctx) + 1
    nb = sum(-(-c // 256) for c in ctx) + 3
    perm = rng.permutation(nb)
    rows_bt, nxt = [], 0
    for c in ctx:
        n = -(-c // 256)
        rows_bt.append(list(perm[nxt:nxt + n]))
        nxt += n
    bt = wl.pad_block_tables(rows_bt, mb)
    kc = wl.normal_bf16(rng, (nb, 256, hkv, D))
    vc = wl.normal_bf16(rng, (nb, 256, hkv, D))
    q = wl.normal_bf16(rng, (B, hq, D))
    cl = np.array(ctx, np.int32)
    o = pkv.attn_decode_paged(to_dev(q, dev), to_dev(kc, dev), to_dev(vc, dev), to_dev(cl, dev), to_dev(bt, dev))
    torch.cuda.synchronize()
    ref = oracle.attn_decode(q, kc.reshape(-1, hkv, D), vc.reshape(-1, hkv, D), cl, bt, hq, hkv)
    out = {"o": o, "ref": ref}
    if nan_canaries:
        kc2, vc2 = kc.copy(), vc.copy()
        used = np.zeros((nb, 256), bool)
        for b, c in enumerate(ctx):
            for j in range(c):
                used[bt[b, j // 256], j % 256] = True
        kc2[~used] = 0x7FC0
        vc2[~used] = 0x7FC0
        out["o_nan"] = pkv.attn_decode_paged(to_dev(q, dev), to_dev(kc2, dev), to_dev(vc2, dev), to_dev(cl, dev),
                                             to_dev(bt, dev))
    if permute:
        p = rng.permutation(nb)
        kc3 = np.empty_like(kc)
        vc3 = np.empty_like(vc)
        kc3[p] = kc
        vc3[p] = vc
        bt3 = np.where(bt >= 0, p[np.maximum(bt, 0)], -1).astype(np.int32)
        out["o_perm"] = pkv.attn_decode_paged(to_dev(q, dev), to_dev(kc3, dev), to_dev(vc3, dev), to_dev(cl, dev),
                                              to_dev(bt3, dev))
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("hq,hkv", [(16, 8), (32, 8), (8, 8), (64, 8), (128, 8)])
def test_decode_small_ragged(dev, hq, hkv):
    ctx = [1, 2, 255, 256, 257, 300, 1000, 4097, 0]
    _say(f"decode contexts {ctx}, {hq}/{hkv} heads, NaN canaries, permuted pool")
    r = _decode_case(dev, ctx, hq, hkv, seed=hq, nan_canaries=True, permute=True)
    got = f64(r["o"])
    check_attn(got[:-1], r["ref"][:-1], "decode small")
    assert np.all(got[-1] == 0.0), "zero-length context must give a zero row"
    assert torch.equal(r["o"], r["o_nan"]), "bytes outside the context changed the output"
    assert torch.equal(r["o"], r["o_perm"]), "physical block placement changed the output"


@pytest.mark.parametrize("hq,hkv", [(32, 8), (16, 8), (8, 1)])
def test_decode_short_contexts_sub_block_splits(dev, hq, hkv):
    """Short contexts at a small batch run in splits of 64 keys (4 chunks of 16 keys),
    not whole blocks: splits that end mid-block, partial chunks, padded ring trips,
    empty splits past the context.  NaN canaries and a permuted pool as above."""
    ctx = [1, 15, 16, 17, 63, 64, 65, 130, 700, 0]
    mb = max(-(-c // 256) for c in ctx) + 1
    # the workspace shows the split length: 16 splits of 64 keys per 4-block row
    need = pkv.decode_workspace_bytes(len(ctx), hq, hkv, mb)
    assert need >= len(ctx) * hq * (mb * 256 // 64) * D * 4, "expected 64-key splits"
    _say(f"decode short contexts {ctx}, {hq}/{hkv} heads, 64-key splits")
    r = _decode_case(dev, ctx, hq, hkv, seed=hq + 2, nan_canaries=True, permute=True)
    got = f64(r["o"])
    check_attn(got[:-1], r["ref"][:-1], "decode sub-block splits")
    assert np.all(got[-1] == 0.0), "zero-length context must give a zero row"
    assert torch.equal(r["o"], r["o_nan"]), "bytes outside the context changed the output"
    assert torch.equal(r["o"], r["o_perm"]), "physical block placement changed the output"


def test_decode_long_context_many_splits(dev):
    ctx = [32768, 20000, 9000]
    _say(f"decode long contexts {ctx}")
    r = _decode_case(dev, ctx, 32, 8, seed=11)
    check_attn(f64(r["o"]), r["ref"], "decode long")


@pytest.mark.parametrize("hq,hkv", [(32, 8), (64, 4)])
def test_decode_longest_context(dev, hq, hkv):
    """Qwen3's longest context (40960 positions, the length of its RoPE table), one short of it,
    and one token: one-block splits, more than 32 of them per sequence (the wide merge), the
    size-ordered grid; every row against the oracle, GQA groups of 4 and 16."""
    ctx = [40960, 40959, 1]
    _say(f"decode contexts {ctx}, {hq}/{hkv} heads")
    r = _decode_case(dev, ctx, hq, hkv, seed=31 + hq)
    check_attn(f64(r["o"]), r["ref"], "decode longest context")


def test_decode_large_batch_short_contexts(dev):
    """1500 sequences: the split-item sort and the grid loop over more items than threads."""
    rng = wl.rng_for(97, 0, 0)
    ctx = [int(c) for c in rng.integers(0, 700, size=1500)]
    ctx[:3] = [0, 1, 699]
    _say("decode 1500 sequences, contexts 0..699, 32/8 heads")
    r = _decode_case(dev, ctx, 32, 8, seed=21)
    got = f64(r["o"])
    live = np.array(ctx) > 0
    check_attn(got[live], r["ref"][live], "decode large batch")
    assert np.all(got[~live] == 0.0)


def test_prefill_2048_short_sequences(dev):
    """2048 sequences of 0-16 new tokens at 32/8 heads (many one-block units, empty sequences
    between them), then 512 of them over paged prefixes of up to 300 keys; every row against
    the oracle."""
    rng = wl.rng_for(93, 2, 0)
    lq = [int(x) for x in rng.integers(0, 17, size=2048)]
    lq[:3] = [0, 1, 16]
    _say("prefill case 1, 2048 sequences of 0-16 tokens, 32/8 heads")
    o, ref, _ = _prefill_case(dev, lq, lq, 32, 8, seed=2048)
    check_attn(f64(o), ref, "prefill 2048 short sequences")
    lq2 = lq[:512]                   # one 256-token block per sequence in the paged pool
    lk = [q + int(p) for q, p in zip(lq2, rng.integers(0, 301, size=512))]
    _say("prefill case 2, 512 sequences of 0-16 tokens over up to 316 keys, 32/8 heads")
    o2, ref2, _ = _prefill_case(dev, lq2, lk, 32, 8, seed=2049, paged=True)
    check_attn(f64(o2), ref2, "prefill 2048 short sequences, paged")


def test_decode_8192_sequences(dev):
    """8192 sequences of 0-64 tokens over a 64-block pool that they share at random (valid, as a
    shared prefix is): the size sort over 8192 split items (16384 workgroups), one-split merges
    and empty rows, every row against the oracle."""
    rng = wl.rng_for(97, 1, 0)
    B, nb = 8192, 64
    ctx = rng.integers(0, 65, size=B).astype(np.int32)
    ctx[:4] = [0, 1, 64, 63]
    bt = np.stack([rng.integers(0, nb, size=B), np.full(B, -1)], 1).astype(np.int32)
    kc = wl.normal_bf16(rng, (nb, 256, 8, D))
    vc = wl.normal_bf16(rng, (nb, 256, 8, D))
    q = wl.normal_bf16(rng, (B, 32, D))
    _say("decode 8192 sequences, contexts 0..64 in a shared 64-block pool, 32/8 heads")
    o = pkv.attn_decode_paged(to_dev(q, dev), to_dev(kc, dev), to_dev(vc, dev), to_dev(ctx, dev), to_dev(bt, dev))
    torch.cuda.synchronize()
    got = f64(o)
    live = ctx > 0
    ref = oracle.attn_decode(q[live], kc.reshape(-1, 8, D), vc.reshape(-1, 8, D), ctx[live], bt[live], 32, 8)
    check_attn(got[live], ref, "decode 8192 sequences")
    assert np.all(got[~live] == 0.0)


def test_prefill_longest_context(dev):
    """One sequence of Qwen3's longest context (40960 tokens) at 32/8 heads, fresh, then its last
    2048 tokens as new queries over the paged cache; rows at both ends, at tile and 2^15
    boundaries, and at random, against the oracle."""
    L = 40960
    rng = wl.rng_for(93, 1, 0)
    pick = [0, 1, 63, 64, 127, 128, 32767, 32768, L - 129, L - 128, L - 2, L - 1]
    rows = [[p, h] for p in pick for h in (0, 31)]
    rows += np.stack([rng.integers(0, L, 96), rng.integers(0, 32, 96)], 1).tolist()
    rows = np.array(rows, np.int64)
    _say(f"prefill case 1, one sequence of {L} tokens, 32/8 heads")
    o, ref, _ = _prefill_case(dev, [L], [L], 32, 8, seed=L, rows=rows)
    check_attn(f64(o)[rows[:, 0], rows[:, 1]], ref, "prefill longest context")
    lq = 2048
    rows2 = [[p, h] for p in (0, 1, 127, 128, 1024, lq - 2, lq - 1) for h in (0, 31)]
    rows2 += np.stack([rng.integers(0, lq, 64), rng.integers(0, 32, 64)], 1).tolist()
    rows2 = np.array(rows2, np.int64)
    _say(f"prefill case 2, {lq} queries over {L} keys, 32/8 heads")
    o2, ref2, _ = _prefill_case(dev, [lq], [L], 32, 8, seed=L + 1, paged=True, rows=rows2)
    check_attn(f64(o2)[rows2[:, 0], rows2[:, 1]], ref2, "prefill longest context, paged")


def test_prefill_long_paged_chunk(dev):
    """A 300-query chunk at the end of a 40960-token context (the largest position), paged."""
    _say("prefill: 300 queries over 40960 paged keys, sampled rows")
    rng = np.random.default_rng(5)
    rows = np.stack([rng.integers(0, 300, 48), rng.integers(0, 32, 48)], 1)
    rows[:2] = [[0, 0], [299, 31]]
    o, ref, _ = _prefill_case(dev, [300], [40960], 32, 8, seed=23, paged=True, rows=rows)
    check_attn(f64(o)[rows[:, 0], rows[:, 1]], ref, "prefill long chunk")


def _pool_workload(dev, w):
    hkv = w.shape.num_kv_heads
    kc = torch.empty((w.num_blocks, 256, hkv, D), dtype=torch.bfloat16, device=dev)
    vc = torch.empty_like(kc)
    wl.fill_normal_bf16_(kc, w.config_id, w.seed, 10)
    wl.fill_normal_bf16_(vc, w.config_id, w.seed, 11)
    return kc, vc


def test_decode_0_6b_workload_full(dev):
    w = wl.paged_decode_0_6b(seed=0)
    _say("decode 0.6B workload: 64 sequences, contexts U[512, 8192]")
    kc, vc = _pool_workload(dev, w)
    q = to_dev(w.q(), dev)
    o = pkv.attn_decode_paged(q, kc, vc, to_dev(w.context_lens, dev), to_dev(w.block_tables, dev))
    torch.cuda.synchronize()
    ref = oracle.attn_decode(bits(q), bits(kc).reshape(-1, 8, D), bits(vc).reshape(-1, 8, D), w.context_lens,
                             w.block_tables, 16, 8)
    check_attn(f64(o), ref, "decode 0.6B")


def test_decode_8b_workload_full(dev):
    """The 8B decode batch (256 sequences, contexts log-U[1024, 32768], 64 sharing an
    8-block prefix): every sequence against the oracle, 32 sequences' blocks copied to
    the host at a time."""
    w = wl.paged_decode_8b(seed=0)
    _say("decode 8B workload: 256 sequences, contexts log-U[1024, 32768], shared prefix; all sequences")
    kc, vc = _pool_workload(dev, w)
    q = to_dev(w.q(), dev)
    o = pkv.attn_decode_paged(q, kc, vc, to_dev(w.context_lens, dev), to_dev(w.block_tables, dev))
    torch.cuda.synchronize()
    got, qh = f64(o), bits(q)
    errs = []
    for s0 in range(0, w.batch, 32):
        seqs = list(range(s0, min(s0 + 32, w.batch)))
        kch, vch, bt = gather_sequences(kc, vc, w.block_tables, seqs, w.context_lens)
        ref = oracle.attn_decode(qh[seqs], kch, vch, w.context_lens[seqs], bt, 32, 8)
        errs.append(np.abs(got[seqs] - ref))
    err = np.concatenate(errs)
    assert np.isfinite(got).all()
    assert err.max() <= 2e-2 and err.mean() <= 2e-3, (err.max(), err.mean())
    _say(f"  max |err| {err.max():.3e}, mean {err.mean():.3e} over {w.batch} sequences")


# ---------------------------------------------------------------------------
# the tiny chain end to end, and decode == prefill row
# ---------------------------------------------------------------------------

def test_tiny_chain_end_to_end(dev, table_dev, table_host):
    _say("tiny chain: qk_norm_rope -> store_kvcache -> prefill -> 4 decode steps")
    w = wl.tiny_chain(seed=0)
    s = w.shape
    q0, k0, v0 = wl.qkv_views(s)
    n = w.qkv.shape[0]
    # GPU
    kc = torch.zeros((w.num_blocks, 256, 8, D), dtype=torch.bfloat16, device=dev)
    vc = torch.zeros_like(kc)
    qkv = to_dev(w.qkv, dev)
    gq, gk = to_dev(w.gamma_q, dev), to_dev(w.gamma_k, dev)
    qo, ko = pkv.qk_norm_rope(qkv[:, q0:k0].view(n, 16, D), qkv[:, k0:v0].view(n, 8, D),
                              to_dev(w.positions, dev), gq, gk, table_dev, s.eps)
    vv = qkv[:, v0:].view(n, 8, D)
    pkv.store_kvcache(ko, vv, kc, vc, to_dev(w.slot_mapping, dev))
    cu = to_dev(w.cu_seqlens, dev)
    o = pkv.attn_prefill_varlen(qo, ko, vv, cu, cu, 300, 300)
    # oracle
    rq = oracle.rmsnorm_rope(w.qkv, 16, D, w.gamma_q, s.eps, w.positions, table_host, col_offset=q0)
    rk = oracle.rmsnorm_rope(w.qkv, 8, D, w.gamma_k, s.eps, w.positions, table_host, col_offset=k0)
    qb, kb = oracle.round_bf16(rq), oracle.round_bf16(rk)
    vb = np.ascontiguousarray(w.qkv[:, v0:]).reshape(n, 8, D)
    ekc = np.zeros((w.num_blocks * 256, 8, D), np.uint16)
    evc = np.zeros_like(ekc)
    oracle.store_kvcache(kb, vb, ekc, evc, w.slot_mapping)
    ref = oracle.attn_prefill(qb, kb, vb, w.cu_seqlens, w.cu_seqlens, 16, 8)
    torch.cuda.synchronize()
    check_attn(f64(o), ref, "chain prefill")
    # the page's integration check: cache rows at the written slots hold k' (within one bf16 ulp)
    got_k = bits(kc).reshape(-1, 8, D)[w.slot_mapping]
    check_ulp(got_k, rk, kb, "cached k'")
    assert np.array_equal(bits(vc).reshape(-1, 8, D)[w.slot_mapping], vb)
    bt = to_dev(w.block_tables, dev)
    for st in w.decode_steps:
        sq = to_dev(st.qkv, dev)
        qd, kd = pkv.qk_norm_rope(sq[:, q0:k0].view(2, 16, D), sq[:, k0:v0].view(2, 8, D),
                                  to_dev(st.positions, dev), gq, gk, table_dev, s.eps)
        pkv.store_kvcache(kd, sq[:, v0:].view(2, 8, D), kc, vc, to_dev(st.slot_mapping, dev))
        od = pkv.attn_decode_paged(qd, kc, vc, to_dev(st.context_lens, dev), bt)
        rqd = oracle.round_bf16(oracle.rmsnorm_rope(st.qkv, 16, D, w.gamma_q, s.eps, st.positions, table_host,
                                                    col_offset=q0))
        rkd = oracle.round_bf16(oracle.rmsnorm_rope(st.qkv, 8, D, w.gamma_k, s.eps, st.positions, table_host,
                                                    col_offset=k0))
        oracle.store_kvcache(rkd, np.ascontiguousarray(st.qkv[:, v0:]).reshape(2, 8, D), ekc, evc, st.slot_mapping)
        refd = oracle.attn_decode(rqd, ekc, evc, st.context_lens, w.block_tables, 16, 8)
        torch.cuda.synchronize()
        check_attn(f64(od), refd, f"chain decode pos {list(st.positions)}")


def test_decode_row_equals_prefill_row(dev):
    _say("decode at position i vs prefill row i (GPU vs GPU)")
    lens = [41, 304, 777]
    hq, hkv = 32, 8
    o, _, inp = _prefill_case(dev, lens, lens, hq, hkv, seed=13, paged=True)
    q, kc, vc, cuq, cuk, bt = inp
    nb = kc.shape[0] // 256
    last = cuq[1:] - 1
    od = pkv.attn_decode_paged(to_dev(np.ascontiguousarray(q[last]), dev), to_dev(kc.reshape(nb, 256, hkv, D), dev),
                               to_dev(vc.reshape(nb, 256, hkv, D), dev), to_dev(np.array(lens, np.int32), dev),
                               to_dev(bt, dev))
    torch.cuda.synchronize()
    err = np.abs(f64(od) - f64(o)[last])
    assert err.max() <= 2e-2, err.max()


@pytest.mark.parametrize("bad_id", [-1, 10 ** 6])
def test_prefill_unusable_block_id_drops_its_keys(dev, bad_id):
    """Case 2 prefill (large enough for the fast pass, 4-wave workgroups) whose block
    tables hold an unusable id (-1, or past the pool) for block 1 of every sequence:
    those 256 keys are never read and drop out of the softmax.  Every query sits past
    block 1, so its result equals a decode over the same table with that entry
    removed and the context shortened by 256 (attention depends only on the set of
    visible keys)."""
    _say(f"prefill case 2 with block id {bad_id} in block 1 of every sequence")
    rng = wl.rng_for(99, 1 if bad_id < 0 else 2, 0)
    hq, hkv, B, lq, lk = 32, 8, 8, 1000, 3000
    nbs = -(-lk // 256)
    nb = B * nbs
    kc = wl.normal_bf16(rng, (nb, 256, hkv, D))
    vc = wl.normal_bf16(rng, (nb, 256, hkv, D))
    q = wl.normal_bf16(rng, (B * lq, hq, D))
    bt = rng.permutation(nb).astype(np.int32).reshape(B, nbs)
    bt_bad = bt.copy()
    bt_bad[:, 1] = bad_id
    cuq, cuk = wl.cu_seqlens([lq] * B), wl.cu_seqlens([lk] * B)
    o = pkv.attn_prefill_varlen(to_dev(q, dev), to_dev(kc, dev), to_dev(vc, dev), to_dev(cuq, dev), to_dev(cuk, dev),
                                lq, lk, block_table=to_dev(bt_bad, dev))
    torch.cuda.synchronize()
    t = np.arange(0, B * lq, 37)
    b, i = t // lq, t % lq
    bt_drop = np.concatenate([bt[:, :1], bt[:, 2:], np.zeros((B, 1), np.int32)], 1)[b]   # block 1 removed
    ctx = (lk - lq + i + 1 - 256).astype(np.int32)
    got = f64(o)[t]                                                                      # [rows, hq, d]
    ref = oracle.attn_decode(q[t], kc.reshape(-1, hkv, D), vc.reshape(-1, hkv, D), ctx, bt_drop, hq, hkv)
    assert np.isfinite(got).all()
    check_attn(got, ref, f"prefill with block id {bad_id}")


def test_decode_unusable_block_ids_drop_their_keys(dev):
    """A block id of -1 or past the pool inside the context: its keys are never read and
    drop out of the softmax (the documented behaviour for invalid metadata).  With the
    bad id in the last block, the result is attention over the keys before it."""
    _say("decode with -1 / out-of-pool block ids in the last block of the context")
    rng = wl.rng_for(98, 0, 0)
    hq, hkv, nb = 32, 8, 12
    kc = wl.normal_bf16(rng, (nb, 256, hkv, D))
    vc = wl.normal_bf16(rng, (nb, 256, hkv, D))
    q = wl.normal_bf16(rng, (3, hq, D))
    bt = np.array([[3, 7, -1, -1], [0, 5, 11, 1000], [2, 9, 4, -1]], np.int32)
    ctx = np.array([700, 1000, 700], np.int32)
    o = pkv.attn_decode_paged(to_dev(q, dev), to_dev(kc, dev), to_dev(vc, dev), to_dev(ctx, dev), to_dev(bt, dev))
    torch.cuda.synchronize()
    kept = np.array([512, 768, 700], np.int32)          # keys before the unusable block (row 2 is valid)
    bt_ok = np.where(bt < 0, 0, np.minimum(bt, nb - 1)).astype(np.int32)
    ref = oracle.attn_decode(q, kc.reshape(-1, hkv, D), vc.reshape(-1, hkv, D), kept, bt_ok, hq, hkv)
    check_attn(f64(o), ref, "decode with unusable blocks")
