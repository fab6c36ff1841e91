"""CPU oracle for the elementwise steps around the attention core: the fused
residual-add + RMSNorm, SiluAndMul, and the Gumbel-max sampler with its
counter-based noise.

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may use it.  numpy float64 throughout, in the
order the pages write each step; no blocking, fusion or reordering.  Shares
no code with the HIP path.

Readings (where the pages leave a step open):
  * add_rms_norm: the pages add in fp32, keep the sum rounded to bf16 as the new
    residual, normalise the fp32 sum, round the normalised value to bf16, then
    multiply by gamma in bf16 ("3.3 Model skeleton and core operators",
    section 2; "同一个 Qwen3，两种写法", section 3.6).  The fp32 add and the two
    bf16 roundings are kept exactly; the mean of squares and the reciprocal
    root are taken in fp64 (the pages' fp32 would only add error).
  * silu_and_mul: silu(gate) * up is evaluated exactly and rounded to bf16 once
    (the pages run it as one compiled elementwise function).
  * Sampler noise: the pages draw E ~ Exp(1) with torch's generator.  Here the
    noise is either given, or drawn from Philox4x32-10 (Salmon, Moraes, Dror,
    Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC 2011) with a fixed
    counter layout, turned into a uniform on (0, 1] and then into Exp(1) by
    inversion, E = -ln(u).
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

from . import bf16_to_f64, round_bf16

# ---------------------------------------------------------------------------
# residual add + RMSNorm  ("3.3 Model skeleton and core operators", section 2;
# "同一个 Qwen3，两种写法", section 3.6)
# ---------------------------------------------------------------------------


def add_rms_norm(x_bits: np.ndarray, residual_bits: Optional[np.ndarray], gamma_bits: np.ndarray,
                 eps: float) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Rows of bf16 bits [T, d].  Returns (y_bits, new_residual_bits, normalised value before ·gamma).

    With residual None this is the plain rms_forward: the input itself is normalised
    and the returned residual is the input unchanged.
    """
    x32 = bf16_to_f64(x_bits).astype(np.float32)
    if residual_bits is None:
        s32 = x32
    else:
        s32 = x32 + bf16_to_f64(residual_bits).astype(np.float32)     # one IEEE fp32 add per element
    new_residual = round_bf16(s32.astype(np.float64))
    s = s32.astype(np.float64)
    var = np.mean(s * s, axis=-1, keepdims=True)
    r = 1.0 / np.sqrt(var + eps)
    normed = s * r
    n_bits = round_bf16(normed)                                         # cast back to bf16
    y = bf16_to_f64(n_bits) * bf16_to_f64(gamma_bits)[None, :]           # bf16 * bf16 is exact in fp64
    return round_bf16(y), new_residual, normed


# ---------------------------------------------------------------------------
# SiluAndMul  ("3.3 Model skeleton and core operators", section 4)
# ---------------------------------------------------------------------------


def silu_and_mul(x_bits: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """x [T, 2I] bf16 bits: front half gate, back half up.  Returns (exact fp64 result, bf16 bits)."""
    x = bf16_to_f64(x_bits)
    half = x.shape[-1] // 2
    gate, up = x[..., :half], x[..., half:]
    silu = gate / (1.0 + np.exp(-gate))
    out = silu * up
    return out, round_bf16(out)


# ---------------------------------------------------------------------------
# Philox4x32-10 and the exponential noise
# ---------------------------------------------------------------------------

PHILOX_M0 = np.uint64(0xD2511F53)
PHILOX_M1 = np.uint64(0xCD9E8D57)
PHILOX_W0 = np.uint32(0x9E3779B9)
PHILOX_W1 = np.uint32(0xBB67AE85)
_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(ctr: np.ndarray, key: np.ndarray) -> np.ndarray:
    """ctr [..., 4] uint32, key [..., 2] uint32 (broadcast) -> [..., 4] uint32.

    Each round multiplies words 0 and 2 by the two round constants into
    (hi, lo) halves and mixes: (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1,
    lo(M0 c0)); the key is bumped by the Weyl constants between rounds.
    """
    c = [np.asarray(ctr[..., i], dtype=np.uint32) for i in range(4)]
    k0 = np.asarray(key[..., 0], dtype=np.uint32).copy()
    k1 = np.asarray(key[..., 1], dtype=np.uint32).copy()
    with np.errstate(over="ignore"):
        for rnd in range(10):
            if rnd > 0:
                k0 = (k0 + PHILOX_W0).astype(np.uint32)
                k1 = (k1 + PHILOX_W1).astype(np.uint32)
            p0 = PHILOX_M0 * c[0].astype(np.uint64)
            p1 = PHILOX_M1 * c[2].astype(np.uint64)
            hi0, lo0 = (p0 >> np.uint64(32)).astype(np.uint32), (p0 & _MASK32).astype(np.uint32)
            hi1, lo1 = (p1 >> np.uint64(32)).astype(np.uint32), (p1 & _MASK32).astype(np.uint32)
            c = [hi1 ^ c[1] ^ k0, lo1, hi0 ^ c[3] ^ k1, lo0]
    return np.stack(c, axis=-1)


def noise_bits(seed: int, offset: int, rows: np.ndarray, cols: np.ndarray) -> np.ndarray:
    """The 32-bit draw for (row, column) pairs (broadcast): Philox counter
    (column // 4, row, offset low 32 bits, offset high 32 bits), key (seed low, seed
    high), output word column % 4."""
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    rows, cols = np.broadcast_arrays(rows, cols)
    ctr = np.stack([(cols >> 2).astype(np.uint32), rows.astype(np.uint32),
                    np.full(rows.shape, offset & 0xFFFFFFFF, np.uint32),
                    np.full(rows.shape, (offset >> 32) & 0xFFFFFFFF, np.uint32)], axis=-1)
    key = np.array([seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF], dtype=np.uint32)
    out = philox4x32_10(ctr, key)
    return np.take_along_axis(out, (cols & 3)[..., None], axis=-1)[..., 0]


def uniform_from_bits(bits: np.ndarray) -> np.ndarray:
    """Top 24 bits of the draw -> (k + 1) / 2^24, uniform on (0, 1] and exact in fp32."""
    return ((np.asarray(bits, dtype=np.uint32) >> np.uint32(8)).astype(np.float64) + 1.0) * 2.0 ** -24


def exp_noise(seed: int, offset: int, num_rows: int, vocab: int) -> np.ndarray:
    """E[b, i] ~ Exp(1) by inversion of the Philox uniform: E = -ln(u)."""
    u = uniform_from_bits(noise_bits(seed, offset, np.arange(num_rows)[:, None], np.arange(vocab)[None, :]))
    return -np.log(u)


# ---------------------------------------------------------------------------
# Sampler  ("3.3 Model skeleton and core operators", section 9)
# ---------------------------------------------------------------------------


def gumbel_max_sample(logits: np.ndarray, temperatures: np.ndarray, seed: int = 0, offset: int = 0,
                      noise: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Tokens argmax_i p_i / E_i per row, in the pages' order: divide the logits by the
    row's temperature, softmax, draw E ~ Exp(1) (given, or Philox), clamp E below at
    1e-10, divide, argmax (first index on ties).  Returns (tokens int64, scores p/E)."""
    lg = np.asarray(logits, dtype=np.float64) / np.asarray(temperatures, dtype=np.float64)[:, None]
    m = lg.max(axis=1, keepdims=True)
    e = np.exp(lg - m)
    p = e / e.sum(axis=1, keepdims=True)
    E = exp_noise(seed, offset, lg.shape[0], lg.shape[1]) if noise is None else np.asarray(noise, np.float64)
    E = np.maximum(E, 1e-10)
    score = p / E
    return np.argmax(score, axis=1).astype(np.int64), score
