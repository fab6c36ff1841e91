"""GPU parity of the elementwise steps around attention: residual add + RMSNorm,
SiluAndMul and the Gumbel-max sampler, against oracle/sublayer.py.

Gates (derived in the comments of each helper):
  * new residual: bit-exact (an fp32 add and one rounding on both sides);
  * RMSNorm y: within one bf16 step of the normalised value times |gamma| plus
    one ulp of y, and >= 99.9% bit-identical;
  * SiluAndMul: within one bf16 ulp of the exact value, >= 99% bit-identical;
  * sampler: the oracle's token, except where the two best scores are closer
    than the kernel's fp32 error bound (then either token is a correct draw).
"""
import numpy as np
import pytest
import torch
from scipy import stats

import oracle
import paged_kv_gqa_amd as pkv
import workloads as wl
from gpu_helpers import bf16_ulp, bits, to_dev
from oracle import sublayer as sl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pkv.load_library()
    return torch.device("cuda:0")


def _say(*a):
    print("[gpu]", *a, flush=True)


# ---------------------------------------------------------------- add + RMSNorm

def _check_rms(y_bits, ref_bits, normed, gamma_bits, what):
    """The kernel's fp32 sum of squares and reciprocal root can move s*r across a
    bf16 rounding boundary: then the rounded normalised value is one bf16 step off,
    which after the product with gamma is ulp(n)|gamma|, plus the final rounding."""
    got = wl.bf16_to_f32(y_bits).astype(np.float64)
    ref = wl.bf16_to_f32(ref_bits).astype(np.float64)
    g = np.abs(wl.bf16_to_f32(gamma_bits).astype(np.float64))[None, :]
    tol = bf16_ulp(normed) * g + bf16_ulp(ref)
    bad = np.abs(got - ref) > tol
    assert not bad.any(), f"{what}: {bad.sum()} values beyond one step (max {np.abs(got - ref).max():.3e})"
    same = np.mean(y_bits == ref_bits)
    assert same >= 0.999, f"{what}: only {same:.5f} bit-identical"


@pytest.mark.parametrize("n_tokens,hidden", [(777, 4096), (333, 1024), (50, 5120), (9, 16384), (21, 520), (5, 8)])
def test_add_rms_norm_matches_oracle(dev, n_tokens, hidden):
    _say(f"add_rms_norm T={n_tokens} hidden={hidden}")
    x, r, g = wl.add_rms_inputs(hidden, n_tokens, hidden)
    xd, rd, gd = to_dev(x, dev), to_dev(r, dev), to_dev(g, dev)
    y, res = pkv.add_rms_norm(xd, rd, gd, 1e-6)
    y0, same = pkv.add_rms_norm(xd, None, gd, 1e-6)
    torch.cuda.synchronize()
    ref_y, ref_res, normed = sl.add_rms_norm(x, r, g, 1e-6)
    assert np.array_equal(bits(res), ref_res), "new residual must be bit-exact"
    _check_rms(bits(y), ref_y, normed, g, "y")
    ref_y0, _, normed0 = sl.add_rms_norm(x, None, g, 1e-6)
    assert same is xd
    _check_rms(bits(y0), ref_y0, normed0, g, "y (no residual)")


@pytest.mark.parametrize("case", range(8))
def test_add_rms_norm_random_shapes(dev, case):
    """Seeded random token counts (log-uniform up to 5000) and widths (multiples of 8 up to
    16384, every lane-count and chunk-count path of the kernel), with and without a residual."""
    rng = wl.rng_for(90, case, 0)
    hidden = 8 * int(rng.integers(1, 2049))
    t = min(int(np.exp(rng.uniform(0, np.log(5001)))), 4_000_000 // hidden)
    _say(f"add_rms_norm random case {case}: T={t} hidden={hidden}")
    x, r, g = wl.add_rms_inputs(1000 + case, t, hidden)
    xd, rd, gd = to_dev(x, dev), to_dev(r, dev), to_dev(g, dev)
    y, res = pkv.add_rms_norm(xd, rd, gd, 1e-6)
    y0, _ = pkv.add_rms_norm(xd, None, gd, 1e-6)
    torch.cuda.synchronize()
    ref_y, ref_res, normed = sl.add_rms_norm(x, r, g, 1e-6)
    assert np.array_equal(bits(res), ref_res), "new residual must be bit-exact"
    _check_rms(bits(y), ref_y, normed, g, "y")
    ref_y0, _, normed0 = sl.add_rms_norm(x, None, g, 1e-6)
    _check_rms(bits(y0), ref_y0, normed0, g, "y (no residual)")


def test_add_rms_norm_in_place(dev):
    _say("add_rms_norm in place")
    x, r, g = wl.add_rms_inputs(3, 300, 4096)
    xd, rd, gd = to_dev(x, dev), to_dev(r, dev), to_dev(g, dev)
    y, res = pkv.add_rms_norm(xd, rd, gd, 1e-6)
    pkv.add_rms_norm(xd, rd, gd, 1e-6, y=xd, residual_out=rd)
    torch.cuda.synchronize()
    assert torch.equal(xd.view(torch.int16), y.view(torch.int16))
    assert torch.equal(rd.view(torch.int16), res.view(torch.int16))


# ---------------------------------------------------------------- SiluAndMul

@pytest.mark.parametrize("n_tokens,inter", [(333, 12288), (64, 3072), (7, 8), (1, 520)])
def test_silu_and_mul_matches_oracle(dev, n_tokens, inter):
    _say(f"silu_and_mul T={n_tokens} I={inter}")
    x = wl.silu_inputs(inter, n_tokens, inter)
    out = pkv.silu_and_mul(to_dev(x, dev))
    torch.cuda.synchronize()
    ref, ref_bits = sl.silu_and_mul(x)
    got_bits = bits(out)
    got = wl.bf16_to_f32(got_bits).astype(np.float64)
    # fp32 evaluation (exp, divide, multiply: a few 2^-24 relative) then one rounding
    bad = np.abs(got - ref) > bf16_ulp(ref)
    assert not bad.any(), f"{bad.sum()} values beyond one bf16 ulp"
    assert np.mean(got_bits == ref_bits) >= 0.99


@pytest.mark.parametrize("case", range(6))
def test_silu_and_mul_random_shapes(dev, case):
    """Seeded random token counts and intermediate widths (multiples of 8 up to 24576)."""
    rng = wl.rng_for(91, case, 0)
    inter = 8 * int(rng.integers(1, 3073))
    t = min(int(np.exp(rng.uniform(0, np.log(3001)))), 2_000_000 // inter)
    _say(f"silu_and_mul random case {case}: T={t} I={inter}")
    x = wl.silu_inputs(2000 + case, t, inter)
    out = pkv.silu_and_mul(to_dev(x, dev))
    torch.cuda.synchronize()
    ref, ref_bits = sl.silu_and_mul(x)
    got_bits = bits(out)
    got = wl.bf16_to_f32(got_bits).astype(np.float64)
    bad = np.abs(got - ref) > bf16_ulp(ref)
    assert not bad.any(), f"{bad.sum()} values beyond one bf16 ulp"
    assert np.mean(got_bits == ref_bits) >= 0.99


def test_silu_and_mul_strided_rows(dev):
    _say("silu_and_mul on a column slice of wider rows")
    x = wl.silu_inputs(5, 40, 1024)
    wide = np.zeros((40, 2048 + 64), np.uint16)
    wide[:, :2048] = x
    xd = to_dev(wide, dev)[:, :2048]
    out_wide = torch.zeros((40, 1024 + 16), dtype=torch.bfloat16, device=xd.device)
    pkv.silu_and_mul(xd, out=out_wide[:, :1024])
    ref = pkv.silu_and_mul(to_dev(x, dev))
    torch.cuda.synchronize()
    assert torch.equal(out_wide[:, :1024].view(torch.int16), ref.view(torch.int16))
    assert out_wide[:, 1024:].float().abs().max().item() == 0.0


# ---------------------------------------------------------------- sampler

def _check_tokens(got, logits_f64, temps, score, what):
    """Accept the oracle's token, or another whose score is within the kernel's error.

    The kernel ranks s_i = (l_i / T) log2(e) - log2(E_i) in fp32: a few roundings of
    2^-24 relative on each term (the product by log2(e)/T, two hardware logarithms,
    the subtraction), so two scores closer than 2^-21 (|l_i/T| + |ln E_i| + 1) summed
    over both tokens (natural-log units) may be ordered either way."""
    want = np.argmax(score, axis=1)
    ls = np.log(score)
    z = logits_f64 / np.asarray(temps, np.float64)[:, None]
    zmax = z.max(axis=1, keepdims=True)
    lnp = z - zmax - np.log(np.exp(z - zmax).sum(axis=1, keepdims=True))
    lnE = lnp - ls
    mism = np.nonzero(got != want)[0]
    for b in mism:
        g, o = int(got[b]), int(want[b])
        assert 0 <= g < score.shape[1], f"{what}: row {b} token {g} out of range"
        tol = 2.0 ** -21 * (abs(z[b, g]) + abs(z[b, o]) + abs(lnE[b, g]) + abs(lnE[b, o]) + 2.0)
        assert ls[b, o] - ls[b, g] <= tol, (f"{what}: row {b} token {g} vs oracle {o}, "
                                            f"score gap {ls[b, o] - ls[b, g]:.3e} > {tol:.3e}")
    assert len(mism) <= max(1, len(got) // 100), f"{what}: {len(mism)} near-ties is implausibly many"


def test_sampler_philox_matches_oracle(dev):
    _say("sampler: 48 rows x 151936 bf16 logits, in-kernel Philox noise")
    lg, temps = wl.sampler_inputs(0, 48)
    got = pkv.sample_gumbel(to_dev(lg, dev), to_dev(temps, dev), seed=1234, offset=7).cpu().numpy()
    lf = wl.bf16_to_f32(lg).astype(np.float64)
    tok, score = sl.gumbel_max_sample(lf, temps.astype(np.float64), seed=1234, offset=7)
    _check_tokens(got, lf, temps, score, "philox")
    # another offset gives other draws for the same logits
    got2 = pkv.sample_gumbel(to_dev(lg, dev), to_dev(temps, dev), seed=1234, offset=8).cpu().numpy()
    tok2, score2 = sl.gumbel_max_sample(lf, temps.astype(np.float64), seed=1234, offset=8)
    _check_tokens(got2, lf, temps, score2, "philox offset 8")


def test_sampler_given_noise_fp32_logits_and_tail(dev):
    _say("sampler: given noise, fp32 logits, vocab 1003 (tail path)")
    rng = wl.rng_for(96, 0, 0)
    B, V, W = 40, 1003, 1004                        # fp32 rows padded to a 16-byte multiple
    lf = (rng.standard_normal((B, V)) * 3).astype(np.float32)
    temps = rng.uniform(0.2, 1.5, B).astype(np.float32)
    E = rng.exponential(size=(B, V)).astype(np.float32)
    temps[0], lf[0, 5], E[0, 5] = 1.0, 0.0, 0.0     # E clamps to 1e-10: token 5 must win row 0
    pad = lambda a: to_dev(np.pad(a, ((0, 0), (0, W - V))), dev)[:, :V]
    got = pkv.sample_gumbel(pad(lf), to_dev(temps, dev), noise=pad(E)).cpu().numpy()
    tok, score = sl.gumbel_max_sample(lf.astype(np.float64), temps.astype(np.float64), noise=E.astype(np.float64))
    assert got[0] == 5 and tok[0] == 5
    _check_tokens(got, lf.astype(np.float64), temps, score, "given noise")
    got_p = pkv.sample_gumbel(pad(lf), to_dev(temps, dev), seed=5).cpu().numpy()
    tok_p, score_p = sl.gumbel_max_sample(lf.astype(np.float64), temps.astype(np.float64), seed=5)
    _check_tokens(got_p, lf.astype(np.float64), temps, score_p, "philox tail")


def test_sampler_distribution_on_gpu(dev):
    """argmax p/E ~ Categorical(p): 100k rows of the same 6 logits, each row its own draw."""
    _say("sampler distribution: 100000 rows x 6 tokens")
    logits = np.array([1.0, 0.0, -1.0, 2.5, 0.5, -3.0], np.float32)
    B = 100_000
    lg = torch.from_numpy(np.tile(np.pad(logits, (0, 2)), (B, 1))).to(dev)[:, :6]    # rows of 8 floats
    T = torch.full((B,), 0.8, dtype=torch.float32, device=dev)
    tok = pkv.sample_gumbel(lg, T, seed=99).cpu().numpy()
    z = logits.astype(np.float64) / np.float64(np.float32(0.8))
    p = np.exp(z) / np.exp(z).sum()
    counts = np.bincount(tok, minlength=6)
    assert counts.sum() == B
    assert stats.chisquare(counts, p * B).pvalue > 1e-4
