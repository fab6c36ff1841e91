"""Brute-force numpy (float64) twin of the attention oracle, for small inputs.

TEST INFRASTRUCTURE ONLY (see the package docstring).

It materialises what the fast paths never build: the full [Tq, Tk] score
matrix over the flat token axis and the block-diagonal, lower-triangular
mask drawn in "同一个 Qwen3，两种写法" section 3.2 (tokens of different
sequences never see each other; inside a sequence query i sees keys up to
its own position).  With fewer queries than keys in a sequence, query i sits
at absolute position Lk - Lq + i ("nano-vllm code walkthrough", "Prefill
stage", case 2).  GQA is written the way the transformers comparison in
"同一个 Qwen3，两种写法" section 3.4 does it: K/V heads are repeated Hq/Hkv
times (contiguous groups) and ordinary multi-head attention follows.
Shares no code with pkv_oracle.c.
"""
from __future__ import annotations

import numpy as np


def flat_causal_mask(cu_q: np.ndarray, cu_k: np.ndarray) -> np.ndarray:
    """Boolean [Tq, Tk] mask over the flat token axes (True = may attend)."""
    cu_q = np.asarray(cu_q, dtype=np.int64)
    cu_k = np.asarray(cu_k, dtype=np.int64)
    Tq, Tk = int(cu_q[-1]), int(cu_k[-1])
    seq_q = np.searchsorted(cu_q, np.arange(Tq), side="right") - 1
    seq_k = np.searchsorted(cu_k, np.arange(Tk), side="right") - 1
    lq = (cu_q[1:] - cu_q[:-1])[seq_q]
    lk = (cu_k[1:] - cu_k[:-1])[seq_q]
    pos_q = (np.arange(Tq) - cu_q[seq_q]) + (lk - lq)      # absolute position of each query
    pos_k = np.arange(Tk) - cu_k[seq_k]
    same = seq_q[:, None] == seq_k[None, :]
    return same & (pos_k[None, :] <= pos_q[:, None])


def repeat_kv(x: np.ndarray, n_rep: int) -> np.ndarray:
    """[T, Hkv, d] -> [T, Hkv*n_rep, d], each kv head copied to its n_rep q heads."""
    T, Hkv, d = x.shape
    return np.broadcast_to(x[:, :, None, :], (T, Hkv, n_rep, d)).reshape(T, Hkv * n_rep, d)


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, cu_q, cu_k, scale: float) -> np.ndarray:
    """softmax(Q K^T * scale + mask) V per head, float64.

    q [Tq, Hq, d], k/v [Tk, Hkv, d] as float arrays; returns [Tq, Hq, d].
    Rows whose mask is empty (no visible key) return 0.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Hq, Hkv = q.shape[1], k.shape[1]
    kk = repeat_kv(k, Hq // Hkv)
    vv = repeat_kv(v, Hq // Hkv)
    mask = flat_causal_mask(cu_q, cu_k)
    out = np.zeros_like(q)
    for h in range(Hq):
        s = (q[:, h, :] @ kk[:, h, :].T) * scale
        s = np.where(mask, s, -np.inf)
        m = np.max(s, axis=1, keepdims=True)
        m = np.where(np.isfinite(m), m, 0.0)
        p = np.exp(s - m)
        l = p.sum(axis=1, keepdims=True)
        out[:, h, :] = np.where(l > 0, (p @ vv[:, h, :]) / np.where(l > 0, l, 1.0), 0.0)
    return out


def gather_paged(cache: np.ndarray, block_table: np.ndarray, lengths, block_size: int) -> np.ndarray:
    """Concatenate each sequence's first lengths[b] logical rows from a paged cache.

    cache is [num_slots, Hkv, d]; logical row j of sequence b is slot
    block_table[b][j // bs] * bs + j % bs.
    """
    rows = []
    for b, L in enumerate(lengths):
        j = np.arange(int(L))
        slots = block_table[b][j // block_size].astype(np.int64) * block_size + j % block_size
        rows.append(cache[slots])
    return np.concatenate(rows, axis=0) if rows else cache[:0]
