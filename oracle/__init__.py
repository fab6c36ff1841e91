"""CPU oracle for the Qwen3 attention-sublayer core.

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  The product
path (``paged_kv_gqa_amd``) never imports it, and this package never
imports the product path.

Two independent implementations live here:

* ``pkv_oracle.c`` (this module's ctypes wrapper): plain loops in fp64,
  OpenMP over independent outputs; the reference for every parity test.
* ``brute`` (numpy, float64): full score matrices with an explicit flat
  block-diagonal causal mask, for small inputs only; used to pin the C code.

Every function cites the page section it follows; the readings taken where
the pages are silent are listed in the C file's header.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pkv_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile pkv_oracle.c with gcc (-O2, OpenMP) into oracle/liboracle.so."""
    if not force and os.path.exists(_LIB_PATH) and os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-fvisibility=hidden",
           "-D_GNU_SOURCE", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P, I32, I64, F64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    lib.orc_round_bf16.argtypes = [P, P, I64]
    lib.orc_round_bf16.restype = None
    lib.orc_bf16_to_double.argtypes = [P, P, I64]
    lib.orc_bf16_to_double.restype = None
    lib.orc_rope_table.argtypes = [P, I32, I32, F64]
    lib.orc_rope_table.restype = ctypes.c_int
    lib.orc_rmsnorm_rope.argtypes = [P, I64, I32, I32, I32, P, F64, P, P, I32, I32, P]
    lib.orc_rmsnorm_rope.restype = ctypes.c_int
    lib.orc_store_kvcache.argtypes = [P, I64, P, I64, P, P, I64, P, I32, I32, I32]
    lib.orc_store_kvcache.restype = ctypes.c_int
    lib.orc_attn_prefill.argtypes = [P, I64, P, I64, P, I64, P, P, I32, I32, I32, I32, F64, P, I32, I32, I64, P, I64,
                                     P]
    lib.orc_attn_prefill.restype = ctypes.c_int
    lib.orc_attn_decode.argtypes = [P, P, P, P, P, I32, I32, I32, I32, I32, I32, I64, F64, P, I32, P]
    lib.orc_attn_decode.restype = ctypes.c_int
    lib.orc_num_threads.argtypes = []
    lib.orc_num_threads.restype = ctypes.c_int
    lib.orc_set_num_threads.argtypes = [I32]
    lib.orc_set_num_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    return int(_load().orc_num_threads())


def set_num_threads(n: int) -> int:
    """Host threads the following oracle calls use; returns the count in force."""
    return int(_load().orc_set_num_threads(int(n)))


# --------------------------------------------------------------------------
# bf16 helpers
# --------------------------------------------------------------------------

def round_bf16(x: np.ndarray) -> np.ndarray:
    """fp64 values -> bf16 bits, round to nearest even (direct, one rounding)."""
    x = _c(x, np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().orc_round_bf16(_p(x), _p(out), x.size)
    return out


def bf16_to_f64(b: np.ndarray) -> np.ndarray:
    b = _c(b, np.uint16)
    out = np.empty(b.shape, dtype=np.float64)
    _load().orc_bf16_to_double(_p(b), _p(out), b.size)
    return out


# --------------------------------------------------------------------------
# RoPE table, QK-Norm + RoPE
# --------------------------------------------------------------------------

def rope_table(max_pos: int = 40960, rot_dim: int = 128, theta: float = 1.0e6) -> np.ndarray:
    """cos/sin table [max_pos, rot_dim] fp32: row p = [cos(p f_i) | sin(p f_i)].

    "3.3 Model skeleton and core operators", section 3 (RoPE table built at init);
    "同一个 Qwen3，两种写法", section 3.5 (one fp32 table for all positions).
    """
    out = np.empty((max_pos, rot_dim), dtype=np.float32)
    rc = _load().orc_rope_table(_p(out), max_pos, rot_dim, float(theta))
    if rc:
        raise ValueError("orc_rope_table rejected its arguments")
    return out


def rmsnorm_rope(x: np.ndarray, n_heads: int, head_dim: int, gamma: np.ndarray, eps: float,
                 positions: np.ndarray, table: np.ndarray, row_stride: Optional[int] = None,
                 col_offset: int = 0, pages_rounding: bool = False) -> np.ndarray:
    """Per-head RMSNorm (QK-Norm) then RoPE, unrounded fp64 [N, n_heads, head_dim].

    x is a bf16 2-D array of rows; the heads start at column ``col_offset``.
    "3.3 Model skeleton and core operators", sections 2, 3 and 8;
    "Nano-vLLM 源码解读 #17 注意力层", section 4.

    ``pages_rounding``: round to bf16 at the three places the pages' code holds a
    bf16 tensor -- the normalised row (cast back before the weight multiply,
    section 2), its product with gamma, and the rotated row (cast to the input
    dtype, section 3) -- instead of leaving the result unrounded.
    """
    x = _c(x, np.uint16)
    assert x.ndim == 2
    n = x.shape[0]
    rs = x.shape[1] if row_stride is None else row_stride
    if col_offset < 0 or col_offset + n_heads * head_dim > rs or (n and rs * (n - 1) + col_offset +
                                                                 n_heads * head_dim > x.size):
        raise ValueError("heads outside the rows of x")
    pos = _c(positions, np.int64)
    tab = _c(table, np.float32)
    g = _c(gamma, np.uint16)
    out = np.empty((n, n_heads, head_dim), dtype=np.float64)
    base = x.ctypes.data + 2 * col_offset
    rc = _load().orc_rmsnorm_rope(ctypes.c_void_p(base), rs, n, n_heads, head_dim, _p(g), float(eps),
                                  _p(pos), _p(tab), tab.shape[0], int(bool(pages_rounding)), _p(out))
    if rc:
        raise ValueError(f"orc_rmsnorm_rope rejected its arguments ({rc})")
    return out


# --------------------------------------------------------------------------
# store_kvcache
# --------------------------------------------------------------------------

def store_kvcache(key: np.ndarray, value: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                  slot_mapping: np.ndarray, key_row_stride: Optional[int] = None,
                  value_row_stride: Optional[int] = None, row_elems: Optional[int] = None) -> None:
    """In-place scatter: row t of key/value -> cache row slot_mapping[t]; -1 skips.

    "3.3 Model skeleton and core operators", section 7.1;
    "Nano-vLLM 源码解读 #17 注意力层", section 5.1.
    Caches are any C-contiguous arrays whose leading dims flatten to slots of
    ``row_elems`` elements.  key/value are 2-D (or more) C-contiguous arrays of
    rows; row strides default to their row length.
    """
    assert k_cache.flags.c_contiguous and v_cache.flags.c_contiguous
    key = np.ascontiguousarray(key)
    value = np.ascontiguousarray(value)
    n = key.shape[0]
    kr = int(np.prod(key.shape[1:])) if key_row_stride is None else key_row_stride
    vr = int(np.prod(value.shape[1:])) if value_row_stride is None else value_row_stride
    D = kr if row_elems is None else row_elems
    eb = key.itemsize
    num_slots = k_cache.size // D
    sm = _c(slot_mapping, np.int32)
    assert sm.shape[0] == n
    rc = _load().orc_store_kvcache(_p(key), kr, _p(value), vr, _p(k_cache), _p(v_cache), num_slots, _p(sm),
                                   n, D, eb)
    if rc:
        raise ValueError("orc_store_kvcache rejected its arguments")


# --------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------

def attn_prefill(q: np.ndarray, k: np.ndarray, v: np.ndarray, cu_seqlens_q: np.ndarray,
                 cu_seqlens_k: np.ndarray, num_q_heads: int, num_kv_heads: int, head_dim: int = 128,
                 scale: Optional[float] = None, block_table: Optional[np.ndarray] = None,
                 block_size: int = 256, rows: Optional[np.ndarray] = None,
                 q_row_stride: Optional[int] = None, k_row_stride: Optional[int] = None,
                 v_row_stride: Optional[int] = None, q_col: int = 0, k_col: int = 0,
                 v_col: int = 0) -> np.ndarray:
    """Varlen causal GQA prefill in fp64.

    Without block_table, k/v hold each sequence's keys as rows cu_seqlens_k[b]..
    (case 1); with it, k/v are the caches (rows = slots) read through the block
    table (case 2).  "3.3 Model skeleton and core operators", section 7.2;
    "nano-vllm code walkthrough", "Prefill stage"; "同一个 Qwen3，两种写法", s3.2.
    Returns [Tq, Hq, d] (or [n_rows, d] when ``rows`` lists (t, h) pairs).
    Raises ValueError when a key a query attends does not exist: a block id
    outside the pool (or -1) among a sequence's first ceil(Lk / block_size)
    table entries, or contiguous key rows past the end of k/v.
    """
    q = _c(q, np.uint16)
    k = _c(k, np.uint16)
    v = _c(v, np.uint16)
    if block_table is not None and k.ndim == 4:      # caches given as [num_blocks, block_size, Hkv, d]
        k = k.reshape(-1, k.shape[2], k.shape[3])
        v = v.reshape(-1, v.shape[2], v.shape[3])
    qs = q_row_stride if q_row_stride is not None else int(np.prod(q.shape[1:]))
    ks = k_row_stride if k_row_stride is not None else int(np.prod(k.shape[1:]))
    vs = v_row_stride if v_row_stride is not None else int(np.prod(v.shape[1:]))
    cq = _c(cu_seqlens_q, np.int32)
    ck = _c(cu_seqlens_k, np.int32)
    B = cq.shape[0] - 1
    if ck.shape[0] != B + 1 or int(cq[-1]) > q.shape[0]:
        raise ValueError("cu_seqlens do not match the inputs")
    for arr, col, stride, heads in ((q, q_col, qs, num_q_heads), (k, k_col, ks, num_kv_heads),
                                    (v, v_col, vs, num_kv_heads)):
        if col < 0 or col + heads * head_dim > stride or stride * max(arr.shape[0] - 1, 0) + col + \
                heads * head_dim > max(arr.size, 1):
            raise ValueError("heads outside the rows of an input")
    sc = head_dim ** -0.5 if scale is None else scale
    bt = None if block_table is None else _c(block_table, np.int32)
    mb = 0 if bt is None else bt.shape[1]
    if rows is None:
        out = np.empty((int(cq[-1]), num_q_heads, head_dim), dtype=np.float64)
        rp, nr = None, -1
    else:
        rows = _c(rows, np.int64).reshape(-1, 2)
        out = np.empty((rows.shape[0], head_dim), dtype=np.float64)
        rp, nr = rows, rows.shape[0]
    n_slots = min(k.shape[0], v.shape[0])
    rc = _load().orc_attn_prefill(ctypes.c_void_p(q.ctypes.data + 2 * q_col), qs,
                                  ctypes.c_void_p(k.ctypes.data + 2 * k_col), ks,
                                  ctypes.c_void_p(v.ctypes.data + 2 * v_col), vs, _p(cq), _p(ck), B,
                                  num_q_heads, num_kv_heads, head_dim, float(sc), _p(bt), mb, block_size,
                                  n_slots, _p(rp), nr, _p(out))
    if rc == -3:
        raise ValueError("orc_attn_prefill: a sequence attends keys that do not exist (block id outside the "
                         "pool, -1, or rows past the end of k/v)")
    if rc:
        raise ValueError(f"orc_attn_prefill rejected its arguments ({rc})")
    return out


def attn_decode(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, context_lens: np.ndarray,
                block_table: np.ndarray, num_q_heads: int, num_kv_heads: int, head_dim: int = 128,
                block_size: int = 256, scale: Optional[float] = None,
                seqs: Optional[np.ndarray] = None) -> np.ndarray:
    """Paged single-token decode in fp64: [B (or len(seqs)), Hq, d].

    "3.3 Model skeleton and core operators", section 7.2;
    "nano-vllm code walkthrough", "Decode Stage".
    The caches are arrays of slot rows ([num_slots, Hkv, d] or any shape that
    flattens to it).  Raises ValueError when a block id among a sequence's first
    ceil(context_len / block_size) table entries is -1 or outside the pool.
    """
    q = _c(q, np.uint16)
    kc = k_cache if (k_cache.flags.c_contiguous and k_cache.dtype == np.uint16) else _c(k_cache, np.uint16)
    vc = v_cache if (v_cache.flags.c_contiguous and v_cache.dtype == np.uint16) else _c(v_cache, np.uint16)
    cl = _c(context_lens, np.int32)
    bt = _c(block_table, np.int32)
    B = cl.shape[0]
    sc = head_dim ** -0.5 if scale is None else scale
    if seqs is None:
        sp, ns, nout = None, -1, B
    else:
        sp = _c(seqs, np.int32)
        ns, nout = sp.shape[0], sp.shape[0]
    out = np.empty((nout, num_q_heads, head_dim), dtype=np.float64)
    if bt.ndim != 2 or bt.shape[0] != B or q.size < B * num_q_heads * head_dim:
        raise ValueError("block_table / q do not match context_lens")
    n_slots = min(kc.size, vc.size) // (num_kv_heads * head_dim)
    rc = _load().orc_attn_decode(_p(q), _p(kc), _p(vc), _p(cl), _p(bt), bt.shape[1], B, num_q_heads,
                                 num_kv_heads, head_dim, block_size, n_slots, float(sc), _p(sp), ns, _p(out))
    if rc == -3:
        raise ValueError("orc_attn_decode: a context reaches a block id that is -1 or outside the pool")
    if rc:
        raise ValueError(f"orc_attn_decode rejected its arguments ({rc})")
    return out
