"""Pins of the sublayer-op oracle (oracle/sublayer.py) against facts it does not
compute itself: published known answers, closed forms, invariances, library
routines on special cases, and the sampler's distribution."""
import numpy as np
import pytest
import torch
from scipy import stats

import oracle
import workloads as wl
from oracle import sublayer as sl


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)


# ---------------------------------------------------------------- Philox / noise

def test_philox_known_answers(golden):
    for c in golden("philox4x32_10_kat.json")["cases"]:
        ctr = np.array([int(x, 16) for x in c["ctr"]], np.uint32)
        key = np.array([int(x, 16) for x in c["key"]], np.uint32)
        got = sl.philox4x32_10(ctr, key)
        assert [f"{int(x):08x}" for x in got] == c["out"]


def test_uniform_ends_are_exact():
    u = sl.uniform_from_bits(np.array([0, 0xFF, 0x100, 0xFFFFFFFF], np.uint32))
    assert list(u) == [2.0 ** -24, 2.0 ** -24, 2.0 ** -23, 1.0]
    assert np.all(u.astype(np.float32).astype(np.float64) == u)     # exact in fp32


def test_exp_noise_is_exp1():
    E = sl.exp_noise(seed=7, offset=0, num_rows=16, vocab=1 << 16).ravel()
    n = E.size
    assert abs(E.mean() - 1.0) < 5 / np.sqrt(n)
    assert abs(E.var() - 1.0) < 10 / np.sqrt(n)
    assert stats.kstest(E, "expon").pvalue > 1e-3
    # other offsets / seeds give independent streams
    E2 = sl.exp_noise(seed=7, offset=1, num_rows=16, vocab=1 << 16).ravel()
    E3 = sl.exp_noise(seed=8, offset=0, num_rows=16, vocab=1 << 16).ravel()
    assert abs(np.corrcoef(E, E2)[0, 1]) < 5 / np.sqrt(n)
    assert abs(np.corrcoef(E, E3)[0, 1]) < 5 / np.sqrt(n)


# ---------------------------------------------------------------- sampler

def _draws(logits_row, temperature, n, seed=3):
    lg = np.broadcast_to(np.asarray(logits_row, np.float64), (n, len(logits_row)))
    tok, _ = sl.gumbel_max_sample(lg, np.full(n, temperature), seed=seed, offset=0)
    return np.bincount(tok, minlength=len(logits_row))


def test_sampler_draws_follow_softmax():
    """argmax p/E ~ Categorical(p): chi-square of 200k draws against softmax(l / T)."""
    logits = np.array([1.0, 0.0, -1.0, 2.5, 0.5, -3.0])
    for T in (1.0, 0.7):
        p = np.exp(logits / T) / np.exp(logits / T).sum()
        counts = _draws(logits, T, 200_000)
        assert stats.chisquare(counts, p * counts.sum()).pvalue > 1e-4


def test_sampler_temperature_limits():
    logits = np.array([0.3, 1.7, 1.2, -0.4])
    assert _draws(logits, 1e-3, 2000)[1] == 2000                 # T -> 0: greedy
    counts = _draws(logits, 1e4, 100_000)                           # T -> inf: uniform
    assert stats.chisquare(counts).pvalue > 1e-4


def test_sampler_given_noise_special_cases():
    lg = np.array([[0.5, 2.0, 1.0, 2.0], [3.0, -1.0, 0.0, 1.0]])
    T = np.ones(2)
    tok, _ = sl.gumbel_max_sample(lg, T, noise=np.ones_like(lg))      # E = 1: argmax of the logits, first on ties
    assert list(tok) == [1, 0]
    p = np.exp(lg - lg.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    tok, score = sl.gumbel_max_sample(lg, T, noise=p)                  # E = p: every score is 1, first index wins
    assert list(tok) == [0, 0] and np.all(score == 1.0)
    noise = np.ones_like(lg)
    noise[0, 0] = 0.0                                                  # clamped to 1e-10: that token wins
    tok, _ = sl.gumbel_max_sample(lg, T, noise=noise)
    assert tok[0] == 0


# ---------------------------------------------------------------- add + RMSNorm

def test_add_rms_constant_row_is_one():
    x = wl.bf16_bits(np.full((2, 64), 3.0, np.float32))
    g = wl.bf16_bits(np.ones(64, np.float32))
    y, res, _ = sl.add_rms_norm(x, None, g, 1e-6)
    assert np.all(wl.bf16_to_f32(y) == 1.0) and np.array_equal(res, x)
    r0 = np.zeros_like(x)
    y2, res2, _ = sl.add_rms_norm(x, r0, g, 1e-6)                      # zero residual == no residual
    assert np.array_equal(y2, y) and np.array_equal(res2, x)


def test_add_rms_scale_invariance_and_permutation():
    x, r, g = wl.add_rms_inputs(0, 8, 256)
    y, res, _ = sl.add_rms_norm(x, r, g, 0.0)
    s4 = lambda b: wl.bf16_bits(wl.bf16_to_f32(b) * np.float32(4.0))
    y4, res4, _ = sl.add_rms_norm(s4(x), s4(r), g, 0.0)
    assert np.array_equal(y4, y) and np.array_equal(res4, s4(res))
    perm = wl.rng_for(95, 0, 0).permutation(256)
    yp, resp, _ = sl.add_rms_norm(x[:, perm], r[:, perm], g[perm], 1e-6)
    y1, res1, _ = sl.add_rms_norm(x, r, g, 1e-6)
    assert np.array_equal(yp, y1[:, perm]) and np.array_equal(resp, res1[:, perm])


def test_add_rms_matches_torch_pieces():
    x, r, g = wl.add_rms_inputs(1, 16, 4096)
    y, res, normed = sl.add_rms_norm(x, r, g, 1e-6)
    xt, rt, gt = _bf16(x), _bf16(r), _bf16(g)
    s = xt.float() + rt.float()
    assert np.array_equal(res, _bits(s.to(torch.bfloat16)))           # new residual: fp32 add, RNE to bf16
    ref = torch.nn.functional.rms_norm(s.double(), (4096,), eps=1e-6).numpy()
    assert np.max(np.abs(normed - ref) / np.abs(ref).clip(1e-30)) < 1e-14
    n_bits = oracle.round_bf16(normed)
    assert np.array_equal(y, _bits(_bf16(n_bits) * gt))                 # bf16 * gamma in torch
    # the pages' structure A (add, store, then a separate norm of the rounded sum) differs only by rounding
    yA, _, _ = sl.add_rms_norm(res, None, g, 1e-6)
    assert np.max(np.abs(wl.bf16_to_f32(yA) - wl.bf16_to_f32(y))) < 0.05


# ---------------------------------------------------------------- SiluAndMul

def test_silu_and_mul_closed_forms_and_torch():
    I = 512
    x = wl.silu_inputs(0, 8, I)
    out, bits = sl.silu_and_mul(x)
    xt = torch.from_numpy(wl.bf16_to_f32(x).astype(np.float64))
    ref = (torch.nn.functional.silu(xt[:, :I]) * xt[:, I:]).numpy()
    assert np.max(np.abs(out - ref)) < 1e-12
    assert np.array_equal(bits, oracle.round_bf16(ref))
    special = wl.bf16_bits(np.array([[0.0, 20.0, -20.0, 1.0, 3.0, 3.0, 3.0, 2.0]], np.float32))
    o, _ = sl.silu_and_mul(special)
    assert o[0, 0] == 0.0
    assert abs(o[0, 1] - 60.0) < 60.0 * 3e-9                          # silu(20) = 20 (1 - 2e-9)
    assert abs(o[0, 2]) < 3 * 20 * 2.1e-9                              # silu(-20) ~ -4e-8
    assert abs(o[0, 3] - 2.0 / (1.0 + np.exp(-1.0))) < 1e-15           # silu(1) * 2
