"""Helpers for the GPU parity tests: device inputs from the seeded generators,
read-back of device bytes, and the accuracy gates.

Gates (written here once, used by every GPU test):
  * store_kvcache / block-table indexing: bit-exact;
  * bf16 attention outputs vs the fp64 oracle: max |err| <= 2e-2 and
    mean |err| <= 2e-3;
  * q', k' (QK-Norm + RoPE, bf16) vs the unrounded oracle: within one bf16
    ulp of the oracle value plus the fp32 evaluation bound of the rotation
    (see rope_tolerance), and at least 99% equal to its correct rounding.
"""
import numpy as np
import torch

import workloads as wl

ATTN_MAX_ABS = 2e-2
ATTN_MEAN_ABS = 2e-3


def to_dev(a: np.ndarray, device="cuda"):
    """numpy array -> torch tensor on the device; uint16 arrays become bfloat16 (same bits)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def bits(t) -> np.ndarray:
    """bf16 (or any 16-bit) torch tensor -> numpy uint16 bit patterns."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f64(t) -> np.ndarray:
    return wl.bf16_to_f32(bits(t)).astype(np.float64)


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |x| (normal range): 2^(floor(log2|x|) - 7)."""
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(ax)) - 7)


def check_attn(got: np.ndarray, ref: np.ndarray, what: str = ""):
    err = np.abs(got.astype(np.float64) - ref)
    assert np.all(np.isfinite(got)), f"{what}: non-finite outputs"
    mx, mean = float(err.max()), float(err.mean())
    assert mx <= ATTN_MAX_ABS, f"{what}: max abs err {mx:.3e} > {ATTN_MAX_ABS}"
    assert mean <= ATTN_MEAN_ABS, f"{what}: mean abs err {mean:.3e} > {ATTN_MEAN_ABS}"
    return mx, mean


def rope_tolerance(ref: np.ndarray) -> np.ndarray:
    """Allowed |gpu - oracle| for q'/k' of shape [..., 128].

    One bf16 ulp of the exact value (the single final rounding), plus the error
    of evaluating norm and rotation in fp32: out_i = y_i c - y_{i+64} s is
    computed from terms as large as the rotated pair, so its absolute fp32
    error scales with the pair's length |(y_i, y_{i+64})| (= the length of
    (out_i, out_{i+64})), not with |out_i|.  About 16 roundings of 2^-24
    relative (norm sum, rsqrt, two scalings, the rotation) give 2^-20 of the
    pair length; the gate allows 2^-19.  Without the second term values born
    of cancellation (|out_i| << pair length) would demand more than fp32 holds.
    """
    half = ref.shape[-1] // 2
    pair = np.sqrt(ref[..., :half] ** 2 + ref[..., half:] ** 2)
    pair = np.concatenate([pair, pair], axis=-1)
    return bf16_ulp(ref) + 2.0 ** -19 * pair


def check_ulp(got_bits: np.ndarray, ref: np.ndarray, rne_bits: np.ndarray, what: str = ""):
    got = wl.bf16_to_f32(got_bits).astype(np.float64)
    err = np.abs(got - ref)
    ok = err <= rope_tolerance(ref)
    assert ok.all(), f"{what}: {np.count_nonzero(~ok)} values beyond one bf16 ulp + fp32 bound (max {err.max():.3e})"
    same = np.mean(got_bits == rne_bits)
    assert same >= 0.99, f"{what}: only {same:.4f} of values equal the correctly rounded oracle"
    return same


def gather_sequences(k_cache, v_cache, block_table: np.ndarray, seqs, context_lens: np.ndarray):
    """Copy the blocks the chosen sequences use to the host as a compact pool.

    Returns (kc, vc, bt) as numpy: kc/vc [n*256, Hkv, 128] uint16 and a block
    table that addresses them, so the oracle can run on a sample of a pool too
    large to copy whole.
    """
    rows, ids = [], []
    for b in seqs:
        nb = -(-int(context_lens[b]) // 256)
        row = [int(x) for x in block_table[b, :nb]]
        rows.append(row)
        ids.extend(row)
    uniq = sorted(set(ids))
    where = {p: i for i, p in enumerate(uniq)}
    idx = torch.tensor(uniq, dtype=torch.int64, device=k_cache.device)
    kc = bits(k_cache.index_select(0, idx)).reshape(len(uniq) * 256, k_cache.shape[2], 128)
    vc = bits(v_cache.index_select(0, idx)).reshape(len(uniq) * 256, v_cache.shape[2], 128)
    bt = wl.pad_block_tables([[where[p] for p in r] for r in rows], block_table.shape[1])
    return kc, vc, bt
