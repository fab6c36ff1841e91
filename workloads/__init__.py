"""Seeded synthetic inputs for the Qwen3 attention-sublayer core.

This module only draws numbers and lays out metadata (lengths, block
tables, slot mappings, cumulative lengths).  It performs none of the
method's arithmetic: no normalisation, no rotation, no attention.  Both
the GPU path and the CPU oracle consume what it produces, so it sits in
a package of its own.

Shapes and value recipes follow the five workloads the attention pages
describe: Qwen3-0.6B (16 q heads / 8 kv heads) and Qwen3-8B (32 / 8)
shapes, head_dim 128, 256-token KV blocks, bf16 values drawn N(0, 1)
("Nano-vLLM 源码解读 #17 注意力层", sections 3 and 7; "同一个 Qwen3，两种写法",
section 2 config table).  Every generator is seeded through
``numpy.random.default_rng([config_id, seed, stream])`` (PCG64).

bf16 values are carried as raw ``uint16`` bit patterns on the host; the
fp32 -> bf16 conversion used to *make* inputs is round-to-nearest-even.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

BLOCK_SIZE = 256
HEAD_DIM = 128
ROPE_THETA = 1.0e6
RMS_EPS = 1.0e-6
MAX_POSITION = 40960


# ----------------------------------------------------------------------------
# bf16 bit helpers (input construction only)
# ----------------------------------------------------------------------------

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 values -> bf16 bit patterns, round-to-nearest-even; NaN -> 0x7FC0."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    r[np.isnan(x)] = 0x7FC0
    return r


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> exact fp32 values."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def rng_for(config_id: int, seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([int(config_id), int(seed), int(stream)])


def normal_bf16(rng: np.random.Generator, shape, scale: float = 1.0) -> np.ndarray:
    return bf16_bits(rng.standard_normal(size=shape, dtype=np.float32) * np.float32(scale))


def gamma_bf16(rng: np.random.Generator, head_dim: int = HEAD_DIM) -> np.ndarray:
    """Norm weight gamma = 1 + 0.05 * N(0, 1), as bf16."""
    g = 1.0 + 0.05 * rng.standard_normal(size=(head_dim,), dtype=np.float32)
    return bf16_bits(g.astype(np.float32))


# ----------------------------------------------------------------------------
# metadata layout helpers
# ----------------------------------------------------------------------------

def cu_seqlens(lengths) -> np.ndarray:
    lengths = np.asarray(lengths, dtype=np.int64)
    out = np.zeros(len(lengths) + 1, dtype=np.int32)
    out[1:] = np.cumsum(lengths)
    return out


def blocks_needed(n_tokens: int, block_size: int = BLOCK_SIZE) -> int:
    return (int(n_tokens) + block_size - 1) // block_size


def slots_for(block_row: np.ndarray, positions: np.ndarray, block_size: int = BLOCK_SIZE) -> np.ndarray:
    """slot = physical block of the logical block holding the position * block_size + offset."""
    positions = np.asarray(positions, dtype=np.int64)
    phys = np.asarray(block_row, dtype=np.int64)[positions // block_size]
    assert np.all(phys >= 0), "position falls in an unallocated logical block"
    return (phys * block_size + positions % block_size).astype(np.int32)


def pad_block_tables(rows: List[List[int]], width: Optional[int] = None) -> np.ndarray:
    width = width if width is not None else max((len(r) for r in rows), default=0)
    bt = np.full((len(rows), max(width, 1)), -1, dtype=np.int32)
    for i, r in enumerate(rows):
        bt[i, : len(r)] = r
    return bt


@dataclass
class Shape:
    num_q_heads: int
    num_kv_heads: int
    head_dim: int = HEAD_DIM
    block_size: int = BLOCK_SIZE
    rope_theta: float = ROPE_THETA
    eps: float = RMS_EPS
    max_position: int = MAX_POSITION

    @property
    def q_size(self) -> int:
        return self.num_q_heads * self.head_dim

    @property
    def kv_size(self) -> int:
        return self.num_kv_heads * self.head_dim

    @property
    def qkv_width(self) -> int:
        return self.q_size + 2 * self.kv_size

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def softmax_scale(self) -> float:
        return self.head_dim ** -0.5


QWEN3_0_6B = Shape(num_q_heads=16, num_kv_heads=8)
QWEN3_8B = Shape(num_q_heads=32, num_kv_heads=8)


def qkv_views(shape: Shape):
    """Column ranges of q, k, v inside one qkv row: split sizes [q_size, kv_size, kv_size]."""
    q0, k0 = 0, shape.q_size
    v0 = k0 + shape.kv_size
    return (q0, k0, v0)


# ----------------------------------------------------------------------------
# Workload 1: tiny two-sequence chain (prefill then 4 decode steps)
# ----------------------------------------------------------------------------

@dataclass
class DecodeStep:
    qkv: np.ndarray            # [B, W] bf16 bits
    positions: np.ndarray      # [B] int64
    slot_mapping: np.ndarray   # [B] int32
    context_lens: np.ndarray   # [B] int32 (including the token written this step)


@dataclass
class TinyChain:
    shape: Shape
    lengths: List[int]
    num_blocks: int
    qkv: np.ndarray                 # [T, W] bf16
    gamma_q: np.ndarray             # [128] bf16
    gamma_k: np.ndarray
    positions: np.ndarray           # [T] int64
    slot_mapping: np.ndarray        # [T] int32
    cu_seqlens: np.ndarray          # [B+1] int32
    block_tables: np.ndarray        # [B, max_blocks] int32, -1 padded
    decode_steps: List[DecodeStep] = field(default_factory=list)


def tiny_chain(seed: int = 0, lengths=(37, 300), n_decode: int = 4, num_blocks: int = 8,
               shape: Shape = QWEN3_0_6B) -> TinyChain:
    rng = rng_for(1, seed, 0)
    perm = rng.permutation(num_blocks).astype(np.int32)
    final_lens = [L + n_decode for L in lengths]
    rows, nxt = [], 0
    for L in final_lens:
        nb = blocks_needed(L, shape.block_size)
        rows.append([int(b) for b in perm[nxt: nxt + nb]])
        nxt += nb
    assert nxt <= num_blocks
    bt = pad_block_tables(rows)
    T = int(sum(lengths))
    qkv = normal_bf16(rng_for(1, seed, 1), (T, shape.qkv_width))
    g = rng_for(1, seed, 2)
    gamma_q, gamma_k = gamma_bf16(g, shape.head_dim), gamma_bf16(g, shape.head_dim)
    positions = np.concatenate([np.arange(L, dtype=np.int64) for L in lengths])
    slot = np.concatenate([slots_for(bt[b], np.arange(L), shape.block_size) for b, L in enumerate(lengths)])
    steps = []
    for j in range(n_decode):
        pos = np.array([L + j for L in lengths], dtype=np.int64)
        steps.append(DecodeStep(
            qkv=normal_bf16(rng_for(1, seed, 10 + j), (len(lengths), shape.qkv_width)),
            positions=pos,
            slot_mapping=np.array([slots_for(bt[b], [p], shape.block_size)[0] for b, p in enumerate(pos)],
                                  dtype=np.int32),
            context_lens=(pos + 1).astype(np.int32)))
    return TinyChain(shape=shape, lengths=list(lengths), num_blocks=num_blocks, qkv=qkv,
                     gamma_q=gamma_q, gamma_k=gamma_k, positions=positions, slot_mapping=slot,
                     cu_seqlens=cu_seqlens(lengths), block_tables=bt, decode_steps=steps)


# ----------------------------------------------------------------------------
# Workload 2: Qwen3-0.6B varlen prefill (8 sequences, lengths U[128, 2048])
# ----------------------------------------------------------------------------

@dataclass
class VarlenPrefill:
    shape: Shape
    lengths: np.ndarray            # [B]
    cu_seqlens: np.ndarray         # [B+1] int32
    num_blocks: int
    block_tables: np.ndarray       # [B, mb] int32
    slot_mapping: np.ndarray       # [T] int32
    positions: np.ndarray          # [T] int64
    seed: int = 0

    @property
    def total_tokens(self) -> int:
        return int(self.cu_seqlens[-1])

    def qkv(self) -> np.ndarray:
        return normal_bf16(rng_for(2, self.seed, 1), (self.total_tokens, self.shape.qkv_width))

    def gammas(self):
        g = rng_for(2, self.seed, 2)
        return gamma_bf16(g), gamma_bf16(g)

    @property
    def flops(self) -> float:
        """Unmasked (i, j) pairs x 4 * head_dim per q head (QK^T and PV)."""
        L = self.lengths.astype(np.float64)
        return float(4 * self.shape.head_dim * self.shape.num_q_heads * np.sum(L * (L + 1) / 2))


def varlen_prefill(seed: int = 0, num_seqs: int = 8, lo: int = 128, hi: int = 2048,
                   num_blocks: int = 4096, shape: Shape = QWEN3_0_6B, lengths=None) -> VarlenPrefill:
    rng = rng_for(2, seed, 0)
    if lengths is None:
        lengths = rng.integers(lo, hi + 1, size=num_seqs)
    lengths = np.asarray(lengths, dtype=np.int64)
    perm = rng_for(2, seed, 3).permutation(num_blocks).astype(np.int32)
    rows, nxt = [], 0
    for L in lengths:
        nb = blocks_needed(int(L), shape.block_size)
        rows.append([int(b) for b in perm[nxt: nxt + nb]])
        nxt += nb
    assert nxt <= num_blocks, "pool too small"
    bt = pad_block_tables(rows)
    positions = np.concatenate([np.arange(L, dtype=np.int64) for L in lengths])
    slot = np.concatenate([slots_for(bt[b], np.arange(L), shape.block_size) for b, L in enumerate(lengths)])
    return VarlenPrefill(shape=shape, lengths=lengths, cu_seqlens=cu_seqlens(lengths), num_blocks=num_blocks,
                         block_tables=bt, slot_mapping=slot, positions=positions, seed=seed)


# ----------------------------------------------------------------------------
# Workloads 3 and 4: paged decode over a pre-filled pool
# ----------------------------------------------------------------------------

@dataclass
class PagedDecode:
    config_id: int
    shape: Shape
    context_lens: np.ndarray       # [B] int32, includes the token decoded this step
    num_blocks: int
    block_tables: np.ndarray       # [B, mb] int32, -1 padded
    shared_seqs: np.ndarray        # indices of sequences mapping onto the shared prefix
    shared_blocks: np.ndarray      # physical ids of the shared prefix blocks
    seed: int = 0

    @property
    def batch(self) -> int:
        return int(len(self.context_lens))

    @property
    def positions(self) -> np.ndarray:
        return (self.context_lens.astype(np.int64) - 1)

    @property
    def slot_mapping(self) -> np.ndarray:
        return np.array([slots_for(self.block_tables[b], [p], self.shape.block_size)[0]
                         for b, p in enumerate(self.positions)], dtype=np.int32)

    def q(self) -> np.ndarray:
        return normal_bf16(rng_for(self.config_id, self.seed, 1),
                           (self.batch, self.shape.num_q_heads, self.shape.head_dim))

    def qkv(self) -> np.ndarray:
        return normal_bf16(rng_for(self.config_id, self.seed, 4), (self.batch, self.shape.qkv_width))

    def gammas(self):
        g = rng_for(self.config_id, self.seed, 2)
        return gamma_bf16(g), gamma_bf16(g)

    def kv_bytes(self, unique: bool = True) -> int:
        """K+V bytes the method must read: context tokens x Hkv x d x 2 bytes x 2.

        With ``unique`` the shared prefix blocks are counted once.
        """
        per_tok = 2 * self.shape.num_kv_heads * self.shape.head_dim * 2
        toks = int(np.sum(self.context_lens.astype(np.int64)))
        if unique and len(self.shared_seqs) > 1:
            toks -= (len(self.shared_seqs) - 1) * len(self.shared_blocks) * self.shape.block_size
        return toks * per_tok

    def algorithmic_bytes(self, unique: bool = True) -> int:
        B, Hq, d = self.batch, self.shape.num_q_heads, self.shape.head_dim
        nblk = int(sum(blocks_needed(int(c), self.shape.block_size) for c in self.context_lens))
        return self.kv_bytes(unique) + B * Hq * d * 2 * 2 + 4 * B + 4 * nblk


def _decode_pool(config_id, seed, ctx, shape, shared_seqs, n_shared_blocks, max_blocks):
    need = 0
    for b, c in enumerate(ctx):
        nb = blocks_needed(int(c), shape.block_size)
        need += nb - (n_shared_blocks if b in shared_seqs else 0)
    need += n_shared_blocks if len(shared_seqs) else 0
    num_blocks = int(math.ceil(1.25 * need))
    perm = rng_for(config_id, seed, 3).permutation(num_blocks).astype(np.int32)
    nxt = 0
    shared = np.array([], dtype=np.int32)
    if len(shared_seqs):
        shared = perm[:n_shared_blocks].copy()
        nxt = n_shared_blocks
    rows = []
    shared_set = set(int(s) for s in shared_seqs)
    for b, c in enumerate(ctx):
        nb = blocks_needed(int(c), shape.block_size)
        if b in shared_set:
            own = perm[nxt: nxt + nb - n_shared_blocks]
            nxt += nb - n_shared_blocks
            rows.append([int(x) for x in shared] + [int(x) for x in own])
        else:
            rows.append([int(x) for x in perm[nxt: nxt + nb]])
            nxt += nb
    assert nxt <= num_blocks
    return num_blocks, pad_block_tables(rows, max_blocks), shared


def paged_decode_0_6b(seed: int = 0, batch: int = 64, lo: int = 512, hi: int = 8192) -> PagedDecode:
    shape = QWEN3_0_6B
    ctx = rng_for(3, seed, 0).integers(lo, hi + 1, size=batch).astype(np.int32)
    mb = blocks_needed(hi, shape.block_size)
    nb, bt, shared = _decode_pool(3, seed, ctx, shape, [], 0, mb)
    return PagedDecode(config_id=3, shape=shape, context_lens=ctx, num_blocks=nb, block_tables=bt,
                       shared_seqs=np.array([], dtype=np.int64), shared_blocks=shared, seed=seed)


def paged_decode_8b(seed: int = 0, batch: int = 256, lo: int = 1024, hi: int = 32768,
                    n_shared_seqs: int = 64, n_shared_blocks: int = 8) -> PagedDecode:
    shape = QWEN3_8B
    r = rng_for(4, seed, 0)
    u = r.uniform(math.log(lo), math.log(hi), size=batch)
    ctx = np.floor(np.exp(u)).astype(np.int64)
    ctx = np.clip(ctx, lo, hi).astype(np.int32)
    # Only sequences whose context has more than the shared prefix plus one token
    # can share it; only full blocks are shared and the decoded token never lands in one.
    eligible = np.nonzero(ctx > n_shared_blocks * shape.block_size)[0]
    n_sh = min(n_shared_seqs, len(eligible))
    shared_seqs = np.sort(rng_for(4, seed, 5).choice(eligible, size=n_sh, replace=False)) if n_sh else \
        np.array([], dtype=np.int64)
    mb = blocks_needed(hi, shape.block_size)
    nb, bt, shared = _decode_pool(4, seed, ctx, shape, list(shared_seqs), n_shared_blocks, mb)
    return PagedDecode(config_id=4, shape=shape, context_lens=ctx, num_blocks=nb, block_tables=bt,
                       shared_seqs=shared_seqs, shared_blocks=shared, seed=seed)


def short_decode_8b(seed: int = 0, batch: int = 64, lo: int = 256, hi: int = 1024) -> PagedDecode:
    """Qwen3-8B-shaped decode over short contexts (U[lo, hi] tokens): the regime in which
    a decode step's kernel launches, not its K/V bytes, set the time."""
    shape = QWEN3_8B
    ctx = rng_for(6, seed, 0).integers(lo, hi + 1, size=batch).astype(np.int32)
    mb = blocks_needed(hi, shape.block_size)
    nb, bt, shared = _decode_pool(6, seed, ctx, shape, [], 0, mb)
    return PagedDecode(config_id=6, shape=shape, context_lens=ctx, num_blocks=nb, block_tables=bt,
                       shared_seqs=np.array([], dtype=np.int64), shared_blocks=shared, seed=seed)


# ----------------------------------------------------------------------------
# Workload 5: Qwen3-8B prefill over a cached shared prefix
# ----------------------------------------------------------------------------

@dataclass
class PrefixPrefill:
    shape: Shape
    num_seqs: int
    prefix_len: int
    total_len: int
    num_blocks: int
    block_tables: np.ndarray      # [B, mb]
    shared_blocks: np.ndarray
    cu_seqlens_q: np.ndarray
    cu_seqlens_k: np.ndarray
    positions: np.ndarray         # [Tq] int64
    slot_mapping: np.ndarray      # [Tq] int32
    seed: int = 0

    @property
    def suffix_len(self) -> int:
        return self.total_len - self.prefix_len

    @property
    def num_q_tokens(self) -> int:
        return self.num_seqs * self.suffix_len

    def qkv(self) -> np.ndarray:
        return normal_bf16(rng_for(5, self.seed, 1), (self.num_q_tokens, self.shape.qkv_width))

    def gammas(self):
        g = rng_for(5, self.seed, 2)
        return gamma_bf16(g), gamma_bf16(g)

    @property
    def flops(self) -> float:
        p = np.arange(self.prefix_len, self.total_len, dtype=np.float64)
        return float(4 * self.shape.head_dim * self.shape.num_q_heads * self.num_seqs * np.sum(p + 1))

    @property
    def store_bytes(self) -> int:
        # per token: the K and V rows read and written (2 x 2 x kv_size bf16) + the 4-byte slot id
        return self.num_q_tokens * (2 * 2 * 2 * self.shape.kv_size + 4)


def prefix_prefill_8b(seed: int = 0, num_seqs: int = 16, prefix_len: int = 2048, total_len: int = 4096,
                      shape: Shape = QWEN3_8B) -> PrefixPrefill:
    bs = shape.block_size
    assert prefix_len % bs == 0
    n_pre = prefix_len // bs
    n_suf = blocks_needed(total_len - prefix_len, bs)
    need = n_pre + num_seqs * n_suf
    num_blocks = int(math.ceil(1.25 * need))
    perm = rng_for(5, seed, 3).permutation(num_blocks).astype(np.int32)
    shared = perm[:n_pre].copy()
    rows, nxt = [], n_pre
    for _ in range(num_seqs):
        rows.append([int(x) for x in shared] + [int(x) for x in perm[nxt: nxt + n_suf]])
        nxt += n_suf
    bt = pad_block_tables(rows)
    Lq = total_len - prefix_len
    positions = np.concatenate([np.arange(prefix_len, total_len, dtype=np.int64)] * num_seqs)
    slot = np.concatenate([slots_for(bt[b], np.arange(prefix_len, total_len), bs) for b in range(num_seqs)])
    return PrefixPrefill(shape=shape, num_seqs=num_seqs, prefix_len=prefix_len, total_len=total_len,
                         num_blocks=num_blocks, block_tables=bt, shared_blocks=shared,
                         cu_seqlens_q=cu_seqlens([Lq] * num_seqs), cu_seqlens_k=cu_seqlens([total_len] * num_seqs),
                         positions=positions, slot_mapping=slot, seed=seed)


# ----------------------------------------------------------------------------
# Device-side pool fill for the large workloads (seeded torch generator)
# ----------------------------------------------------------------------------

def fill_normal_bf16_(tensor, config_id: int, seed: int, stream: int, chunk_elems: int = 1 << 27):
    """Fill a bf16 torch tensor in place with N(0,1) values from a seeded torch.Generator.

    Values are drawn as fp32 on the tensor's device and rounded to bf16 by
    torch's conversion (round-to-nearest-even).  Used for KV pools too big to
    draw on the host; the oracle reads the resulting bytes back.
    """
    import torch
    g = torch.Generator(device=tensor.device)
    g.manual_seed((int(config_id) * 1_000_003 + int(seed)) * 1_000_003 + int(stream))
    flat = tensor.view(-1)
    n = flat.numel()
    for s in range(0, n, chunk_elems):
        e = min(n, s + chunk_elems)
        flat[s:e].copy_(torch.randn(e - s, generator=g, device=tensor.device, dtype=torch.float32))
    return tensor


# ----------------------------------------------------------------------------
# inputs of the elementwise steps around the attention core (Qwen3-8B sizes,
# "同一个 Qwen3，两种写法", section 2 config table: hidden 4096, intermediate
# 12288, vocab 151936)
# ----------------------------------------------------------------------------

HIDDEN_8B = 4096
INTERMEDIATE_8B = 12288
VOCAB = 151936


def add_rms_inputs(seed: int, n_tokens: int, hidden: int = HIDDEN_8B):
    """(x, residual, gamma) bf16 bits: the sublayer output x ~ N(0, 1), the residual
    stream ~ N(0, 3^2) (it accumulates over layers), gamma = 1 + 0.05 N(0, 1)."""
    rng = rng_for(6, seed, 0)
    x = normal_bf16(rng, (n_tokens, hidden))
    residual = normal_bf16(rng, (n_tokens, hidden), scale=3.0)
    return x, residual, gamma_bf16(rng, hidden)


def silu_inputs(seed: int, n_tokens: int, intermediate: int = INTERMEDIATE_8B):
    """gate_up rows [T, 2I] bf16 bits ~ N(0, 2^2): gate in the front half, up in the back."""
    return normal_bf16(rng_for(7, seed, 0), (n_tokens, 2 * intermediate), scale=2.0)


def sampler_inputs(seed: int, num_rows: int, vocab: int = VOCAB):
    """(logits bf16 bits [B, V], temperatures fp32 [B]).

    Logits ~ N(0, 2^2) with 16 favoured tokens per row raised by U(4, 12), so each
    row has a few likely tokens and a long tail.  Temperatures U(0.3, 1.5), and
    every 8th row 0.05 (close to greedy)."""
    rng = rng_for(8, seed, 0)
    lg = rng.standard_normal(size=(num_rows, vocab), dtype=np.float32) * np.float32(2.0)
    fav = np.stack([rng.choice(vocab, size=16, replace=False) for _ in range(num_rows)])
    lg[np.arange(num_rows)[:, None], fav] += rng.uniform(4.0, 12.0, size=fav.shape).astype(np.float32)
    temps = rng.uniform(0.3, 1.5, size=num_rows).astype(np.float32)
    temps[::8] = np.float32(0.05)
    return bf16_bits(lg), temps
