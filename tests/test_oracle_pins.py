"""Pins for the CPU oracle: each test ties it to something other than itself.

Pins used: values the pages print (tests/golden), closed forms, library
routines for special cases (torch float64 rms_norm and scaled-dot-product
attention, numpy complex multiplication for a plane rotation, numpy fancy
indexing for the scatter), invariants (causality, permutation of physical
blocks, decode == prefill row), and the independent numpy brute force.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import brute
import workloads as wl

D = 128


def _f64(b):
    return wl.bf16_to_f32(b).astype(np.float64)


# ---------------------------------------------------------------------------
# widths and sizes (printed on the pages)
# ---------------------------------------------------------------------------

def test_widths_and_sizes(golden):
    g = golden("widths_w1.json")
    s = wl.QWEN3_0_6B
    e = g["qwen3_0_6b"]
    assert (s.q_size, s.kv_size, s.qkv_width, s.group) == (e["q_size"], e["kv_size"], e["qkv_width"], e["group"])
    assert wl.qkv_views(s) == (0, 2048, 3072)
    assert s.num_q_heads * s.head_dim == e["o_flat_width"]
    s8, e8 = wl.QWEN3_8B, g["qwen3_8b"]
    assert (s8.qkv_width, s8.group) == (e8["qkv_width"], e8["group"])
    per_tok = 2 * e8["num_layers"] * s8.num_kv_heads * s8.head_dim * 2
    assert per_tok == e8["kv_bytes_per_token_all_layers"] == 144 * 1024
    assert per_tok * 256 == e8["kv_bytes_per_block_all_layers"] == 36 * 1024 * 1024
    tab = oracle.rope_table(g["rope_table"]["max_position"], g["rope_table"]["rotary_dim"], 1e6)
    assert tab.nbytes == g["rope_table"]["bytes_fp32"]


# ---------------------------------------------------------------------------
# bf16 rounding
# ---------------------------------------------------------------------------

def test_round_bf16_known_values():
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -30, -2.5, 0.0, -0.0,
                     2 ** -140, 3.0e38, 1e39, float("inf"), float("nan")])
    exp = np.array([0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xC020, 0x0000, 0x8000,
                    0x0000, 0x7F62, 0x7F80, 0x7F80, 0x7FC0], dtype=np.uint16)
    got = oracle.round_bf16(vals)
    # 3.0e38 rounds to the nearest bf16 (0x7F62 = 3.0023e38)
    assert wl.bf16_to_f32(np.array([0x7F62], dtype=np.uint16))[0] == pytest.approx(3.0e38, rel=4e-3)
    np.testing.assert_array_equal(got, exp)


def test_round_bf16_matches_fp32_path_on_fp32_values():
    x = np.random.default_rng(7).standard_normal(200000).astype(np.float32) * 37.0
    np.testing.assert_array_equal(oracle.round_bf16(x.astype(np.float64)), wl.bf16_bits(x))


# ---------------------------------------------------------------------------
# RoPE table
# ---------------------------------------------------------------------------

def test_rope_table_closed_forms():
    tab = oracle.rope_table(40960, D, 1e6)
    np.testing.assert_array_equal(tab[0, :64], 1.0)
    np.testing.assert_array_equal(tab[0, 64:], 0.0)
    # column 0 has frequency theta^0 = 1 exactly: the angle is the position itself
    p = np.arange(40960)
    np.testing.assert_array_equal(tab[:, 0], np.cos(p.astype(np.float64)).astype(np.float32))
    np.testing.assert_array_equal(tab[:, 64], np.sin(p.astype(np.float64)).astype(np.float32))
    # cos^2 + sin^2 = 1 up to fp32 rounding
    np.testing.assert_allclose(tab[:, :64].astype(np.float64) ** 2 + tab[:, 64:].astype(np.float64) ** 2, 1.0,
                               atol=4e-7)


def test_rope_table_against_pages_torch_code():
    """Re-run the table construction the pages print, in torch fp32.

    torch's fp32 pow/cos are not correctly rounded, so agreement is to the
    angle error an fp32 frequency can carry (grows with position).
    """
    max_pos = 40960
    inv_freq = 1.0 / (1e6 ** (torch.arange(0, D, 2).float() / D))
    t = torch.arange(max_pos).float()
    freqs = torch.einsum("i,j->ij", t, inv_freq)
    ref = torch.cat((freqs.cos(), freqs.sin()), dim=-1).numpy()
    tab = oracle.rope_table(max_pos, D, 1e6)
    np.testing.assert_allclose(tab[:64], ref[:64], atol=1e-5)
    np.testing.assert_allclose(tab, ref, atol=1e-2)


# ---------------------------------------------------------------------------
# QK-Norm (RMSNorm over head_dim) and RoPE
# ---------------------------------------------------------------------------

def _one_head(x_f32, gamma_f32, pos, eps=1e-6):
    x = wl.bf16_bits(np.asarray(x_f32, np.float32).reshape(1, -1))
    g = wl.bf16_bits(np.asarray(gamma_f32, np.float32))
    tab = oracle.rope_table(max(int(pos) + 1, 2), D, 1e6)
    return oracle.rmsnorm_rope(x, 1, D, g, eps, np.array([pos]), tab)[0, 0]


@pytest.mark.parametrize("c", [2.0 ** -10, 0.5, 3.0, -7.0])
def test_rmsnorm_constant_input_closed_form(c):
    """RMSNorm(c * 1) = c / sqrt(c^2 + eps) * gamma; position 0 rotates by nothing."""
    y = _one_head(np.full(D, c), np.ones(D), 0)
    np.testing.assert_allclose(y, c / math.sqrt(c * c + 1e-6), rtol=1e-12)


def test_rmsnorm_unit_mean_square_and_gamma():
    x = np.where(np.arange(D) % 3 == 0, 1.0, -1.0)
    gamma = wl.bf16_to_f32(wl.bf16_bits(1 + 0.05 * np.random.default_rng(1).standard_normal(D).astype(np.float32)))
    y = _one_head(x, gamma, 0)
    np.testing.assert_allclose(y, x / math.sqrt(1 + 1e-6) * gamma, rtol=1e-12)


def test_rmsnorm_matches_torch_library():
    rng = np.random.default_rng(3)
    x = wl.bf16_bits(rng.standard_normal((6, 4 * D)).astype(np.float32) * 2)
    g = wl.bf16_bits(1 + 0.05 * rng.standard_normal(D).astype(np.float32))
    tab = oracle.rope_table(8, D, 1e6)
    got = oracle.rmsnorm_rope(x, 4, D, g, 1e-6, np.zeros(6, np.int64), tab)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(_f64(x).reshape(6, 4, D)), (D,),
                                       weight=torch.from_numpy(_f64(g)), eps=1e-6).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)


def test_rmsnorm_scale_invariance():
    rng = np.random.default_rng(4)
    x = rng.standard_normal(D).astype(np.float32)
    y1 = _one_head(x, np.ones(D), 0)
    y2 = _one_head(x * 64.0, np.ones(D), 0)      # power-of-two scale keeps bf16 inputs exact
    np.testing.assert_allclose(y1, y2, rtol=1e-5)


def test_rope_is_complex_rotation():
    """RoPE on pairs (i, i+64) is multiplication of x_i + j x_{i+64} by exp(j angle)."""
    rng = np.random.default_rng(5)
    n = 9
    x = wl.bf16_bits(rng.standard_normal((n, 3 * D)).astype(np.float32))
    g = wl.bf16_bits(1 + 0.05 * rng.standard_normal(D).astype(np.float32))
    pos = rng.integers(0, 40960, size=n)
    tab = oracle.rope_table(40960, D, 1e6)
    got = oracle.rmsnorm_rope(x, 3, D, g, 1e-6, pos, tab)
    y = torch.nn.functional.rms_norm(torch.from_numpy(_f64(x).reshape(n, 3, D)), (D,),
                                     weight=torch.from_numpy(_f64(g)), eps=1e-6).numpy()
    rot = tab[pos][:, None, :64].astype(np.float64) + 1j * tab[pos][:, None, 64:].astype(np.float64)
    z = (y[..., :64] + 1j * y[..., 64:]) * rot
    np.testing.assert_allclose(got[..., :64], z.real, rtol=0, atol=1e-12)
    np.testing.assert_allclose(got[..., 64:], z.imag, rtol=0, atol=1e-12)


def test_rope_rotate_half_form_and_norms():
    """The transformers rotate_half form with duplicated 128-wide cos/sin gives the same vector;
    each rotated pair keeps its length; position 0 is the identity."""
    rng = np.random.default_rng(6)
    x = wl.bf16_bits(rng.standard_normal((5, D)).astype(np.float32))
    ones = wl.bf16_bits(np.ones(D, np.float32))
    tab = oracle.rope_table(4096, D, 1e6)
    pos = np.array([0, 1, 17, 1000, 4095])
    got = oracle.rmsnorm_rope(x, 1, D, ones, 1e-6, pos, tab)[:, 0]
    y = oracle.rmsnorm_rope(x, 1, D, ones, 1e-6, np.zeros(5, np.int64), tab)[:, 0]
    np.testing.assert_array_equal(got[0], y[0])
    cos = np.concatenate([tab[pos, :64]] * 2, axis=1).astype(np.float64)
    sin = np.concatenate([tab[pos, 64:]] * 2, axis=1).astype(np.float64)
    rh = np.concatenate([-y[:, 64:], y[:, :64]], axis=1)
    np.testing.assert_allclose(got, y * cos + rh * sin, atol=1e-12)
    np.testing.assert_allclose(got[:, :64] ** 2 + got[:, 64:] ** 2, y[:, :64] ** 2 + y[:, 64:] ** 2,
                               rtol=1e-6)


def test_rope_relative_position_property():
    """<R_p q, R_s k> depends only on p - s (small positions, so fp32 angles are accurate)."""
    rng = np.random.default_rng(8)
    xq = wl.bf16_bits(rng.standard_normal((1, D)).astype(np.float32))
    xk = wl.bf16_bits(rng.standard_normal((1, D)).astype(np.float32))
    ones = wl.bf16_bits(np.ones(D, np.float32))
    tab = oracle.rope_table(512, D, 1e6)

    def dot(p, s):
        a = oracle.rmsnorm_rope(xq, 1, D, ones, 1e-6, np.array([p]), tab)[0, 0]
        b = oracle.rmsnorm_rope(xk, 1, D, ones, 1e-6, np.array([s]), tab)[0, 0]
        return float(a @ b)

    base = dot(7, 3)
    for delta in (1, 10, 100, 400):
        assert dot(7 + delta, 3 + delta) == pytest.approx(base, abs=2e-4)
    assert abs(dot(7, 3) - dot(7, 5)) > 1e-3       # and it does depend on the offset


def test_pages_rounding_worked_example():
    """Pages-rounding mode rounds the normalised row to bf16, then its product with gamma,
    then the rotated row.  Worked by hand for x = [3, 1, 1, ..., 1] at position 0 (no
    rotation), gamma_0 = 1 + 2^-7: mean square (9 + 127) / 128 = 1.0625, so
    n_0 = 3 / sqrt(1.0625 + 1e-6) = 2.91043..., which rounds (bf16 steps of 2^-6 in [2, 4))
    to 186 * 2^-6 = 2.90625; 2.90625 * (1 + 2^-7) = 2.92896 rounds to 187 * 2^-6 = 2.921875.
    Rounded once instead, 2.91043 * (1 + 2^-7) = 2.93317 -> 188 * 2^-6 = 2.9375: the two
    pipelines differ here by one bf16 step.  The other elements: n = 0.97014 -> 0.96875
    (248 * 2^-8), times gamma 1 stays 0.96875."""
    x = np.ones(D, np.float32)
    x[0] = 3.0
    g = np.ones(D, np.float32)
    g[0] = 1.0 + 2.0 ** -7
    xb = wl.bf16_bits(x.reshape(1, -1))
    gb = wl.bf16_bits(g)
    tab = oracle.rope_table(4, D, 1e6)
    pages = oracle.rmsnorm_rope(xb, 1, D, gb, 1e-6, np.array([0]), tab, pages_rounding=True)[0, 0]
    once = oracle.rmsnorm_rope(xb, 1, D, gb, 1e-6, np.array([0]), tab)[0, 0]
    assert pages[0] == 2.921875
    assert np.all(pages[1:] == 0.96875)
    assert once[0] == pytest.approx(3.0 / math.sqrt(1.0625 + 1e-6) * (1 + 2.0 ** -7), rel=1e-14)
    assert wl.bf16_to_f32(oracle.round_bf16(once[:1]))[0] == 2.9375
    # constant input with gamma 1.5: n = 1/sqrt(1 + 1e-6) rounds to 1.0, so y = 1.5 exactly
    c = oracle.rmsnorm_rope(wl.bf16_bits(np.ones((1, D), np.float32)), 1, D,
                            wl.bf16_bits(np.full(D, 1.5, np.float32)), 1e-6, np.array([0]), tab,
                            pages_rounding=True)[0, 0]
    assert np.all(c == 1.5)


def _pages_torch_code(x_bits, n_heads, gamma_bits, eps, positions, table):
    """The pages' own code, run with torch on the CPU: rms_forward ("3.3 Model skeleton and
    core operators" section 2) then apply_rotary_emb (section 3) with the fp32 table."""
    x = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).reshape(x_bits.shape[0], n_heads, D)
    w = torch.from_numpy(gamma_bits.view(np.int16)).view(torch.bfloat16)
    xf = x.float()
    var = xf.pow(2).mean(dim=-1, keepdim=True)
    xf.mul_(torch.rsqrt(var + eps))
    y = xf.to(torch.bfloat16).mul_(w)
    cos, sin = torch.from_numpy(table[positions]).unsqueeze(1).chunk(2, dim=-1)
    x1, x2 = torch.chunk(y.float(), 2, dim=-1)
    out = torch.cat((x1 * cos - x2 * sin, x2 * cos + x1 * sin), dim=-1).to(torch.bfloat16)
    return out.view(torch.int16).numpy().view(np.uint16)


def test_pages_rounding_matches_the_pages_torch_code():
    """The pages compute the mean square, the root and the rotation in fp32, the oracle in
    fp64; the bf16 results agree except where an fp32 rounding moves a value across a bf16
    rounding boundary (then by one bf16 step)."""
    rng = np.random.default_rng(12)
    n, heads = 400, 8
    x = wl.bf16_bits((2.5 * rng.standard_normal((n, heads * D))).astype(np.float32))
    g = wl.bf16_bits(1 + 0.05 * rng.standard_normal(D).astype(np.float32))
    pos = rng.integers(0, 40960, n)
    tab = oracle.rope_table(40960, D, 1e6)
    ref = _pages_torch_code(x, heads, g, 1e-6, pos, tab)
    got = oracle.rmsnorm_rope(x, heads, D, g, 1e-6, pos, tab, pages_rounding=True)
    got_bits = oracle.round_bf16(got)
    np.testing.assert_array_equal(wl.bf16_to_f32(got_bits).astype(np.float64), got)   # already bf16 values
    ref = ref.reshape(got_bits.shape)
    same = np.mean(got_bits == ref)
    assert same >= 0.999, same
    # Where they differ, an fp32 rounding moved a value across a bf16 boundary: the
    # normalised row or its product with gamma by one bf16 step (at most one step of the
    # rotated pair's length after the rotation, |cos|, |sin| <= 1), or the result itself
    # by one step; where x1 cos - x2 sin cancels far below its terms, the fp32 rotation's
    # own error (a few 2^-24 of the pair's length) adds to that.
    def step(a):
        return np.exp2(np.floor(np.log2(np.maximum(np.abs(a), 2.0 ** -126))) - 7)
    r = wl.bf16_to_f32(ref).astype(np.float64)
    pair = np.sqrt(got[..., :64] ** 2 + got[..., 64:] ** 2)
    pair = np.concatenate([pair, pair], axis=-1)
    assert np.all(np.abs(got - r) <= step(r) + 2 * step(pair) + 2.0 ** -19 * pair)
    # At position 0 (no rotation) the output is the bf16 product with gamma itself:
    # differences are single bf16 steps.
    z = np.zeros(n, np.int64)
    ref0 = _pages_torch_code(x, heads, g, 1e-6, z, tab).reshape(got_bits.shape)
    got0 = oracle.round_bf16(oracle.rmsnorm_rope(x, heads, D, g, 1e-6, z, tab, pages_rounding=True))
    assert np.mean(got0 == ref0) >= 0.999
    r0 = wl.bf16_to_f32(ref0).astype(np.float64)
    assert np.all(np.abs(wl.bf16_to_f32(got0).astype(np.float64) - r0) <= step(r0))


# ---------------------------------------------------------------------------
# store_kvcache scatter
# ---------------------------------------------------------------------------

def test_scatter_skeleton_w3(golden):
    g = golden("scatter_skeleton_w3.json")
    src = np.array(g["src"], dtype=np.float32)
    dst_k = np.zeros((g["N"], g["D"]), np.float32)
    dst_v = np.zeros_like(dst_k)
    oracle.store_kvcache(src, src, dst_k, dst_v, np.array(g["slot"], np.int32))
    np.testing.assert_array_equal(dst_k, np.array(g["expected_dst"], np.float32))


def test_store_kvcache_w4(golden):
    g = golden("store_kvcache_w4.json")
    N, nkv, hd = g["N"], g["num_kv_heads"], g["head_dim"]
    base = np.arange(nkv * hd).reshape(1, nkv, hd)
    key = (np.arange(N).reshape(N, 1, 1) * 10 + base).astype(np.float32)
    value = key + 100
    kc = np.zeros(g["cache_shape"], np.float32)
    vc = np.zeros(g["cache_shape"], np.float32)
    oracle.store_kvcache(key, value, kc, vc, np.array(g["slot_mapping"], np.int32))
    np.testing.assert_array_equal(kc.reshape(-1, nkv * hd), np.array(g["expected_k_cache_rows"], np.float32))
    np.testing.assert_array_equal(vc.reshape(-1, nkv * hd)[0], np.array(g["expected_v_cache_slot0"], np.float32))


def test_store_kvcache_matches_index_assignment():
    """The pages' PyTorch equivalent: k_cache.view(-1, D)[slot_mapping] = key.view(N, D) (valid slots)."""
    rng = np.random.default_rng(9)
    N, Dr, slots = 300, 1024, 2048
    qkv = rng.integers(0, 65535, size=(N, 4096), dtype=np.uint16)
    sm = rng.permutation(slots)[:N].astype(np.int32)
    sm[rng.random(N) < 0.1] = -1
    kc = rng.integers(0, 65535, size=(slots // 256, 256, 8, 128), dtype=np.uint16)
    vc = kc.copy()
    ek, ev = kc.copy().reshape(-1, Dr), vc.copy().reshape(-1, Dr)
    ok = sm >= 0
    ek[sm[ok]] = qkv[ok, 2048:3072]
    ev[sm[ok]] = qkv[ok, 3072:4096]
    key = qkv[:, 2048:]        # row stride 4096 handled by explicit strides below
    oracle.store_kvcache(np.ascontiguousarray(qkv[:, 2048:3072]), np.ascontiguousarray(qkv[:, 3072:]), kc, vc, sm)
    np.testing.assert_array_equal(kc.reshape(-1, Dr), ek)
    np.testing.assert_array_equal(vc.reshape(-1, Dr), ev)
    del key


# ---------------------------------------------------------------------------
# softmax / single attention row
# ---------------------------------------------------------------------------

def _decode_one(q_vec, keys, vals, scale=1.0):
    """Run the decode oracle for one sequence of len(keys) keys, d = len(q_vec), 1 head."""
    d = len(q_vec)
    n = len(keys)
    bs = 256
    nblk = max(1, -(-n // bs))
    kc = np.zeros((nblk * bs, 1, d), np.uint16)
    vc = np.zeros_like(kc)
    kc[:n, 0] = wl.bf16_bits(np.asarray(keys, np.float32).reshape(n, d))
    vc[:n, 0] = wl.bf16_bits(np.asarray(vals, np.float32).reshape(n, d))
    q = wl.bf16_bits(np.asarray(q_vec, np.float32)).reshape(1, 1, d)
    bt = np.arange(nblk, dtype=np.int32).reshape(1, -1)
    return oracle.attn_decode(q, kc, vc, np.array([n], np.int32), bt, 1, 1, head_dim=d, block_size=bs,
                              scale=scale)[0, 0]


def test_online_softmax_worked_example_w5(golden):
    g = golden("online_softmax_w5.json")
    s, v, pr = g["s"], g["v"], g["printed"]
    # O with scalar values
    o = _decode_one([1.0], [[x] for x in s], [[x] for x in v])
    assert round(o[0], 3) == pytest.approx(pr["O"], abs=1e-9)
    # weights: one-hot values return the weight vector itself
    w = _decode_one([1.0, 0, 0, 0], [[x, 0, 0, 0] for x in s], np.eye(4))
    np.testing.assert_allclose(np.round(w, 3), pr["weights"], atol=1e-12)
    assert abs(w.sum() - 1.0) < 1e-12
    # the largest score has e^0 = 1, so l = 1 / its weight
    assert round(1.0 / w[int(np.argmax(s))], 3) == pytest.approx(pr["l"], abs=1e-9)
    # the printed two-block figures are consistent with the whole-row result:
    # block A rescaled to block B's max contributes l_A and Obar_A, and the totals match
    m = max(s)
    lA = sum(math.exp(x - m) for x in pr["block_A"])
    oA = sum(math.exp(x - m) * vv for x, vv in zip(pr["block_A"], v[:2]))
    assert round(math.exp(max(pr["block_A"]) - m), 3) == pytest.approx(pr["rescale_factor"], abs=1e-9)
    assert round(lA, 3) == pytest.approx(pr["rescaled_l_of_A"], abs=1e-9)
    assert round(oA, 3) == pytest.approx(pr["rescaled_Obar_of_A"], abs=1e-9)


def test_single_key_returns_value_exactly_and_rows_sum_to_one():
    rng = np.random.default_rng(10)
    q = rng.standard_normal(D)
    v = wl.bf16_to_f32(wl.bf16_bits(rng.standard_normal(D).astype(np.float32)))
    o = _decode_one(q, [rng.standard_normal(D)], [v], scale=D ** -0.5)
    np.testing.assert_array_equal(o, v.astype(np.float64))
    keys = rng.standard_normal((700, D))
    o1 = _decode_one(q, keys, np.ones((700, D)), scale=D ** -0.5)
    assert np.max(np.abs(o1 - 1.0)) < 1e-12


# ---------------------------------------------------------------------------
# prefill / decode against library attention and the brute force
# ---------------------------------------------------------------------------

def _rand_bf16(rng, shape):
    return wl.bf16_bits(rng.standard_normal(shape).astype(np.float32))


def test_prefill_matches_torch_sdpa_per_sequence():
    rng = np.random.default_rng(11)
    lens = [1, 37, 130, 64]
    Hq, Hkv = 16, 8
    cu = wl.cu_seqlens(lens)
    T = int(cu[-1])
    q, k, v = _rand_bf16(rng, (T, Hq, D)), _rand_bf16(rng, (T, Hkv, D)), _rand_bf16(rng, (T, Hkv, D))
    got = oracle.attn_prefill(q, k, v, cu, cu, Hq, Hkv)
    for b, L in enumerate(lens):
        s0 = cu[b]
        qt = torch.from_numpy(_f64(q[s0:s0 + L])).permute(1, 0, 2)[None]
        kt = torch.from_numpy(_f64(k[s0:s0 + L])).permute(1, 0, 2)[None]
        vt = torch.from_numpy(_f64(v[s0:s0 + L])).permute(1, 0, 2)[None]
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=D ** -0.5,
                                                               enable_gqa=True)
        np.testing.assert_allclose(got[s0:s0 + L], ref[0].permute(1, 0, 2).numpy(), atol=1e-12)


def test_prefill_matches_brute_force_and_gqa_equals_repeated_mha():
    rng = np.random.default_rng(12)
    lens = [37, 300]
    Hq, Hkv = 16, 8
    cu = wl.cu_seqlens(lens)
    T = int(cu[-1])
    q, k, v = _rand_bf16(rng, (T, Hq, D)), _rand_bf16(rng, (T, Hkv, D)), _rand_bf16(rng, (T, Hkv, D))
    got = oracle.attn_prefill(q, k, v, cu, cu, Hq, Hkv)
    ref = brute.attention(_f64(q), _f64(k), _f64(v), cu, cu, D ** -0.5)
    assert np.max(np.abs(got - ref)) < 1e-12
    # GQA vs explicit repeat_kv + MHA: same arithmetic, bit-identical
    k_rep = np.ascontiguousarray(np.repeat(k, Hq // Hkv, axis=1))
    v_rep = np.ascontiguousarray(np.repeat(v, Hq // Hkv, axis=1))
    mha = oracle.attn_prefill(q, k_rep, v_rep, cu, cu, Hq, Hq)
    np.testing.assert_array_equal(got, mha)


def test_causal_mask_zeros_and_no_cross_sequence_leak():
    rng = np.random.default_rng(13)
    lens = [50, 70]
    cu = wl.cu_seqlens(lens)
    T = int(cu[-1])
    q, k, v = _rand_bf16(rng, (T, 4, D)), _rand_bf16(rng, (T, 2, D)), _rand_bf16(rng, (T, 2, D))
    base = oracle.attn_prefill(q, k, v, cu, cu, 4, 2)
    # overwrite the keys/values after position 20 of sequence 0 and all of sequence 1
    k2, v2 = k.copy(), v.copy()
    k2[21:] = _rand_bf16(rng, k2[21:].shape)
    v2[21:] = _rand_bf16(rng, v2[21:].shape)
    pert = oracle.attn_prefill(q, k2, v2, cu, cu, 4, 2)
    np.testing.assert_array_equal(base[:21], pert[:21])
    assert np.max(np.abs(base[21:50] - pert[21:50])) > 1e-3
    # sequence 1 must not see sequence 0: change sequence 0 entirely
    k3, v3 = k.copy(), v.copy()
    k3[:50] = _rand_bf16(rng, k3[:50].shape)
    v3[:50] = _rand_bf16(rng, v3[:50].shape)
    np.testing.assert_array_equal(oracle.attn_prefill(q, k3, v3, cu, cu, 4, 2)[50:], base[50:])
    # flat mask shape: block diagonal with lower triangles, as drawn on the page
    m = brute.flat_causal_mask(wl.cu_seqlens([3, 2, 2]), wl.cu_seqlens([3, 2, 2]))
    exp = np.zeros((7, 7), bool)
    for s0, L in ((0, 3), (3, 2), (5, 2)):
        exp[s0:s0 + L, s0:s0 + L] = np.tril(np.ones((L, L), bool))
    np.testing.assert_array_equal(m, exp)


def _paged_from_rows(rng, k_rows, v_rows, lens, num_blocks, bs=256):
    """Scatter each sequence's logical rows into a permuted block pool; return caches and table."""
    Hkv = k_rows.shape[1]
    perm = rng.permutation(num_blocks)
    kc = _rand_bf16(rng, (num_blocks * bs, Hkv, D))      # garbage everywhere else
    vc = _rand_bf16(rng, (num_blocks * bs, Hkv, D))
    rows, nxt, off = [], 0, 0
    for L in lens:
        nb = -(-L // bs)
        rows.append(list(perm[nxt:nxt + nb]))
        nxt += nb
    bt = wl.pad_block_tables(rows)
    for b, L in enumerate(lens):
        slots = wl.slots_for(bt[b], np.arange(L), bs)
        kc[slots] = k_rows[off:off + L]
        vc[slots] = v_rows[off:off + L]
        off += L
    return kc, vc, bt


def test_prefix_prefill_rows_equal_full_prefill_rows():
    rng = np.random.default_rng(14)
    Lk, Lq = [300, 513], [40, 257]
    Hq, Hkv = 8, 2
    cuk, cuq = wl.cu_seqlens(Lk), wl.cu_seqlens(Lq)
    Tk = int(cuk[-1])
    q_full = _rand_bf16(rng, (Tk, Hq, D))
    k, v = _rand_bf16(rng, (Tk, Hkv, D)), _rand_bf16(rng, (Tk, Hkv, D))
    full = oracle.attn_prefill(q_full, k, v, cuk, cuk, Hq, Hkv)
    kc, vc, bt = _paged_from_rows(rng, k, v, Lk, 8)
    sel = np.concatenate([np.arange(cuk[b + 1] - Lq[b], cuk[b + 1]) for b in range(2)])
    part = oracle.attn_prefill(q_full[sel], kc, vc, cuq, cuk, Hq, Hkv, block_table=bt)
    np.testing.assert_array_equal(part, full[sel])
    # and the brute force agrees on the bottom-right alignment
    ref = brute.attention(_f64(q_full[sel]), _f64(brute.gather_paged(kc, bt, Lk, 256)),
                          _f64(brute.gather_paged(vc, bt, Lk, 256)), cuq, cuk, D ** -0.5)
    assert np.max(np.abs(part - ref)) < 1e-12


def test_decode_equals_prefill_row_and_block_permutation_invariance():
    rng = np.random.default_rng(15)
    L = [41, 304, 1]
    Hq, Hkv = 16, 8
    cu = wl.cu_seqlens(L)
    T = int(cu[-1])
    q = _rand_bf16(rng, (T, Hq, D))
    k, v = _rand_bf16(rng, (T, Hkv, D)), _rand_bf16(rng, (T, Hkv, D))
    full = oracle.attn_prefill(q, k, v, cu, cu, Hq, Hkv)
    kc, vc, bt = _paged_from_rows(rng, k, v, L, 8)
    last = cu[1:] - 1
    dec = oracle.attn_decode(np.ascontiguousarray(q[last]), kc, vc, np.array(L, np.int32), bt, Hq, Hkv)
    np.testing.assert_array_equal(dec, full[last])
    # permute physical blocks: same logical content, relabelled table
    nblk = kc.shape[0] // 256
    p = rng.permutation(nblk)
    kc2 = kc.reshape(nblk, 256, Hkv, D)[np.argsort(p)].reshape(kc.shape)
    vc2 = vc.reshape(nblk, 256, Hkv, D)[np.argsort(p)].reshape(vc.shape)
    bt2 = np.where(bt >= 0, p[np.maximum(bt, 0)], -1).astype(np.int32)
    dec2 = oracle.attn_decode(np.ascontiguousarray(q[last]), kc2, vc2, np.array(L, np.int32), bt2, Hq, Hkv)
    np.testing.assert_array_equal(dec, dec2)
    # a context of zero tokens gives a zero row
    z = oracle.attn_decode(np.ascontiguousarray(q[last[:1]]), kc, vc, np.array([0], np.int32), bt[:1], Hq, Hkv)
    np.testing.assert_array_equal(z, 0.0)


# ---------------------------------------------------------------------------
# the tiny chain (workload 1) end to end, oracle only
# ---------------------------------------------------------------------------

def test_tiny_chain_oracle_end_to_end():
    w = wl.tiny_chain(seed=0)
    s = w.shape
    tab = oracle.rope_table(s.max_position, D, s.rope_theta)
    q0, k0, v0 = wl.qkv_views(s)
    kc = np.zeros((w.num_blocks * 256, s.num_kv_heads, D), np.uint16)
    vc = np.zeros_like(kc)
    qn = oracle.rmsnorm_rope(w.qkv, s.num_q_heads, D, w.gamma_q, s.eps, w.positions, tab, col_offset=q0)
    kn = oracle.rmsnorm_rope(w.qkv, s.num_kv_heads, D, w.gamma_k, s.eps, w.positions, tab, col_offset=k0)
    qb, kb = oracle.round_bf16(qn), oracle.round_bf16(kn)
    vb = np.ascontiguousarray(w.qkv[:, v0:]).reshape(-1, s.num_kv_heads, D)
    oracle.store_kvcache(kb, vb, kc, vc, w.slot_mapping)
    # the page's integration check: cache rows at the written slots hold the recomputed k
    np.testing.assert_array_equal(kc[w.slot_mapping], kb)
    np.testing.assert_array_equal(vc[w.slot_mapping], vb)
    o = oracle.attn_prefill(qb, kb, vb, w.cu_seqlens, w.cu_seqlens, s.num_q_heads, s.num_kv_heads)
    assert o.reshape(o.shape[0], -1).shape == (337, 2048)
    # first row of each sequence sees one key: output equals v exactly (per q head's kv head)
    for b in range(2):
        t = w.cu_seqlens[b]
        np.testing.assert_array_equal(o[t], _f64(np.repeat(vb[t], 2, axis=0)))
    # prefill over the paged cache reproduces the contiguous prefill
    op = oracle.attn_prefill(qb, kc, vc, w.cu_seqlens, w.cu_seqlens, s.num_q_heads, s.num_kv_heads,
                             block_table=w.block_tables)
    np.testing.assert_array_equal(op, o)
    # decode steps: write the new token, then attend over the cache
    for st in w.decode_steps:
        qd = oracle.round_bf16(oracle.rmsnorm_rope(st.qkv, s.num_q_heads, D, w.gamma_q, s.eps, st.positions, tab,
                                                   col_offset=q0))
        kd = oracle.round_bf16(oracle.rmsnorm_rope(st.qkv, s.num_kv_heads, D, w.gamma_k, s.eps, st.positions,
                                                   tab, col_offset=k0))
        vd = np.ascontiguousarray(st.qkv[:, v0:]).reshape(-1, s.num_kv_heads, D)
        oracle.store_kvcache(kd, vd, kc, vc, st.slot_mapping)
        od = oracle.attn_decode(qd, kc, vc, st.context_lens, w.block_tables, s.num_q_heads, s.num_kv_heads)
        assert od.shape == (2, 16, 128)
        assert np.all(np.isfinite(od))


def test_results_do_not_depend_on_the_thread_count():
    """Each output row is computed by one thread with its own accumulators, so one host
    thread and all of them give identical bits (prefill, decode and QK-Norm + RoPE)."""
    w = wl.tiny_chain(seed=2)
    s = w.shape
    q0, k0, v0 = wl.qkv_views(s)
    table = oracle.rope_table(4096, 128, s.rope_theta)
    n = w.qkv.shape[0]
    q = np.ascontiguousarray(w.qkv[:, q0:k0]).reshape(n, s.num_q_heads, 128)
    k = np.ascontiguousarray(w.qkv[:, k0:v0]).reshape(n, s.num_kv_heads, 128)
    v = np.ascontiguousarray(w.qkv[:, v0:]).reshape(n, s.num_kv_heads, 128)
    kc = np.zeros((w.num_blocks * 256, s.num_kv_heads, 128), np.uint16)
    vc = np.zeros_like(kc)
    oracle.store_kvcache(k, v, kc, vc, w.slot_mapping)
    ctx = np.array(w.lengths, np.int32)

    def run():
        return (oracle.attn_prefill(q, k, v, w.cu_seqlens, w.cu_seqlens, s.num_q_heads, s.num_kv_heads),
                oracle.attn_decode(q[np.cumsum(w.lengths) - 1], kc, vc, ctx, w.block_tables, s.num_q_heads,
                                   s.num_kv_heads),
                oracle.rmsnorm_rope(w.qkv, s.num_q_heads, 128, w.gamma_q, s.eps, w.positions % 4096, table,
                                    col_offset=q0))

    prev = oracle.num_threads()
    try:
        assert oracle.set_num_threads(1) == 1
        one = run()
    finally:
        oracle.set_num_threads(prev)
    assert oracle.num_threads() == prev
    for a, b in zip(one, run()):
        assert np.array_equal(a, b)
