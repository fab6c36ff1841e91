"""paged_kv_gqa_amd -- the Qwen3 attention-sublayer core on MI355X (gfx950).

A thin ctypes binding over ``libpkv.so`` (HIP kernels + C ABI declared in
``include/pkv.h``).  The functions below only marshal torch tensors into
pointers, strides and sizes; every step runs in the HIP kernels.  There is no
fallback: if the library is missing or cannot be loaded, every call raises.

Entry points mirror the calls the attention pages describe
("3.3 Model skeleton and core operators", sections 3, 7.1, 7.2, 8):

* ``rope_cache_build``   -- the fp32 cos/sin table, once
* ``qk_norm_rope``       -- q_norm / k_norm then rotary_emb(positions, q, k)
* ``store_kvcache``      -- store_kvcache(key, value, k_cache, v_cache, slot_mapping)
* ``qk_norm_rope_store`` -- the two steps above in one pass (rotated k and v go
                            straight to their cache rows)
* ``attn_prefill_varlen``-- flash_attn_varlen_func(q, k, v, cu_seqlens_q, cu_seqlens_k,
                            max_seqlen_q, max_seqlen_k, softmax_scale, causal, block_table)
* ``attn_decode_paged``  -- flash_attn_with_kvcache(q, k_cache, v_cache, cache_seqlens,
                            block_table, softmax_scale, causal)
* ``add_rms_norm``       -- RMSNorm with the residual add folded in (add_rms_forward)
* ``silu_and_mul``       -- SiluAndMul
* ``sample_gumbel``      -- the sampler: argmax softmax(logits / T) / Exp(1) noise
* ``DecodeStep``         -- the decode step (QK-Norm + RoPE + scatter, then paged
                            decode) over static buffers, eager or replayed from
                            HIP graphs captured per batch bucket
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpkv.so")
HEAD_DIM = 128
BLOCK_SIZE = 256

PKV_OK = 0
_STATUS = {-1: "invalid argument", -2: "unsupported", -3: "launch failed", -4: "workspace"}

#: every symbol include/pkv.h declares
EXPORTED = ("pkv_last_error", "pkv_version", "pkv_rope_cache_build", "pkv_qk_norm_rope",
            "pkv_qk_norm_rope_store", "pkv_store_kvcache", "pkv_attn_prefill_varlen", "pkv_attn_prefill_workspace_bytes",
            "pkv_attn_decode_workspace_bytes", "pkv_attn_decode_paged", "pkv_decode_step_workspace_bytes",
            "pkv_decode_step", "pkv_decode_graph_create", "pkv_decode_graph_bucket", "pkv_decode_graph_launch",
            "pkv_decode_graph_destroy", "pkv_add_rms_norm", "pkv_silu_and_mul", "pkv_sample_gumbel",
            "pkv_attn_decode_paged_noalloc")

#: pkv_decode_step_desc.flags bit: the caller pads rows [batch, bucket) itself before a graph launch
PKV_DECODE_CALLER_PADS = 1

#: the batch ladder the decode graphs are captured for
GRAPH_BUCKETS = (1, 2, 4, 8, 16, 32, 64, 128, 256, 512)


class DecodeStepDesc(ctypes.Structure):
    """Mirror of pkv_decode_step_desc (include/pkv.h), field for field."""
    _fields_ = [("qkv", ctypes.c_void_p), ("qkv_row_stride", ctypes.c_int64), ("q_out", ctypes.c_void_p),
                ("o", ctypes.c_void_p), ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
                ("num_blocks", ctypes.c_int64), ("positions", ctypes.c_void_p), ("slot_mapping", ctypes.c_void_p),
                ("context_lens", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
                ("max_blocks_per_seq", ctypes.c_int32), ("max_batch", ctypes.c_int32),
                ("q_norm_weight", ctypes.c_void_p), ("k_norm_weight", ctypes.c_void_p),
                ("cos_sin_cache", ctypes.c_void_p), ("max_position", ctypes.c_int32), ("eps", ctypes.c_float),
                ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("softmax_scale", ctypes.c_float), ("flags", ctypes.c_int32),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t)]

_lib = None


class PkvError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} failed ({code}: {_STATUS.get(code, '?')}): {msg}")
        self.code = code


def load_library(path: str = LIB_PATH):
    """Load libpkv.so and declare its C signatures.  Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run `python -m paged_kv_gqa_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(path)
    P, I32, I64, F32, F64, SZ = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                                 ctypes.c_double, ctypes.c_size_t)
    lib.pkv_last_error.argtypes = []
    lib.pkv_last_error.restype = ctypes.c_char_p
    lib.pkv_version.argtypes = []
    lib.pkv_version.restype = ctypes.c_int
    lib.pkv_rope_cache_build.argtypes = [P, I32, I32, F64, P]
    lib.pkv_rope_cache_build.restype = ctypes.c_int
    lib.pkv_qk_norm_rope.argtypes = [P, I64, P, I64, P, P, P, I32, I32, I32, I32, P, P, F32, P, I32, P]
    lib.pkv_qk_norm_rope.restype = ctypes.c_int
    lib.pkv_qk_norm_rope_store.argtypes = [P, I64, P, I64, P, I64, P, P, P, P, I64, P, P, I32, I32, I32, I32, P,
                                           P, F32, P, I32, P]
    lib.pkv_qk_norm_rope_store.restype = ctypes.c_int
    lib.pkv_store_kvcache.argtypes = [P, I64, P, I64, P, P, I64, P, I32, I32, I32, I32, P]
    lib.pkv_store_kvcache.restype = ctypes.c_int
    lib.pkv_attn_prefill_varlen.argtypes = [P, I64, P, I64, P, I64, P, P, P, I32, I32, I32, I32, I32, I32, I32,
                                            F32, I32, P, I32, I32, I64, P, SZ, P]
    lib.pkv_attn_prefill_varlen.restype = ctypes.c_int
    lib.pkv_attn_prefill_workspace_bytes.argtypes = [I32, I32, I32, I32, I32, I32, I32]
    lib.pkv_attn_prefill_workspace_bytes.restype = SZ
    lib.pkv_attn_decode_workspace_bytes.argtypes = [I32, I32, I32, I32, I32, I32]
    lib.pkv_attn_decode_workspace_bytes.restype = SZ
    lib.pkv_attn_decode_paged.argtypes = [P, P, P, P, P, P, I32, I32, I32, I32, I32, I32, I64, F32, P, SZ, P]
    lib.pkv_attn_decode_paged_noalloc.argtypes = [P, P, P, P, P, P, I32, I32, I32, I32, I32, I32, I64, F32, P]
    lib.pkv_attn_decode_paged_noalloc.restype = ctypes.c_int
    lib.pkv_attn_decode_paged.restype = ctypes.c_int
    lib.pkv_add_rms_norm.argtypes = [P, P, P, P, P, I32, I32, F32, P]
    lib.pkv_add_rms_norm.restype = ctypes.c_int
    lib.pkv_silu_and_mul.argtypes = [P, I64, P, I64, I32, I32, P]
    lib.pkv_silu_and_mul.restype = ctypes.c_int
    lib.pkv_sample_gumbel.argtypes = [P, I64, I32, P, P, I64, ctypes.c_uint64, ctypes.c_uint64, P, I32, I32, P]
    lib.pkv_sample_gumbel.restype = ctypes.c_int
    DP = ctypes.POINTER(DecodeStepDesc)
    lib.pkv_decode_step_workspace_bytes.argtypes = [I32, I32, I32, I32, I32, I32]
    lib.pkv_decode_step_workspace_bytes.restype = SZ
    lib.pkv_decode_step.argtypes = [DP, I32, P]
    lib.pkv_decode_step.restype = ctypes.c_int
    lib.pkv_decode_graph_create.argtypes = [DP, ctypes.POINTER(I32), I32, ctypes.POINTER(P)]
    lib.pkv_decode_graph_create.restype = ctypes.c_int
    lib.pkv_decode_graph_bucket.argtypes = [P, I32]
    lib.pkv_decode_graph_bucket.restype = I32
    lib.pkv_decode_graph_launch.argtypes = [P, I32, P]
    lib.pkv_decode_graph_launch.restype = ctypes.c_int
    lib.pkv_decode_graph_destroy.argtypes = [P]
    lib.pkv_decode_graph_destroy.restype = None
    _lib = lib
    return lib


def _check(fn: str, rc: int):
    if rc != PKV_OK:
        raise PkvError(fn, rc, _lib.pkv_last_error().decode(errors="replace"))


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _rows(x, heads: int, name: str) -> int:
    """Validate a [N, heads, 128] bf16 view (the pages' stride asserts) and return its row stride."""
    import torch
    if x.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16, got {x.dtype}")
    if x.dim() != 3 or x.shape[1] != heads or x.shape[2] != HEAD_DIM:
        raise ValueError(f"{name} must be [N, {heads}, {HEAD_DIM}], got {tuple(x.shape)}")
    if x.shape[0] > 1 and (x.stride(2) != 1 or x.stride(1) != HEAD_DIM):
        raise ValueError(f"{name} needs stride(-1) == 1 and stride(1) == head_dim, got {x.stride()}")
    if x.shape[0] <= 1:
        return max(x.stride(0), heads * HEAD_DIM)
    return x.stride(0)


def _i32(t, name):
    import torch
    if t.dtype != torch.int32 or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous int32 tensor")
    return t


def _same_device(ref, **named):
    """Every tensor given must live on the GPU that holds ``ref`` (the kernels get raw pointers)."""
    if ref.device.type != "cuda":
        raise ValueError(f"inputs must be GPU tensors, got {ref.device}")
    for name, t in named.items():
        if t is not None and t.device != ref.device:
            raise ValueError(f"{name} is on {t.device}, the inputs on {ref.device}")


def _out(t, shape, ref, name):
    """A caller-supplied output must be exactly the contiguous bf16 tensor the kernel writes."""
    import torch
    if t.dtype != torch.bfloat16 or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous bfloat16 tensor of shape {tuple(shape)}, got "
                         f"{t.dtype} {tuple(t.shape)}{'' if t.is_contiguous() else ' (not contiguous)'}")
    if t.device != ref.device:
        raise ValueError(f"{name} is on {t.device}, the inputs on {ref.device}")
    return t


def _norm_params(q_norm_weight, k_norm_weight, cos_sin_cache, ref):
    import torch
    for name, w in (("q_norm_weight", q_norm_weight), ("k_norm_weight", k_norm_weight)):
        if w.dtype != torch.bfloat16 or w.numel() != HEAD_DIM or not w.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bfloat16 tensor of {HEAD_DIM} elements")
    if cos_sin_cache.dtype != torch.float32 or cos_sin_cache.dim() != 2 or cos_sin_cache.shape[1] != HEAD_DIM \
            or not cos_sin_cache.is_contiguous():
        raise ValueError(f"cos_sin_cache must be a contiguous float32 [max_position, {HEAD_DIM}] table")
    _same_device(ref, q_norm_weight=q_norm_weight, k_norm_weight=k_norm_weight, cos_sin_cache=cos_sin_cache)


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------

def rope_cache_build(max_position: int = 40960, rotary_dim: int = HEAD_DIM, theta: float = 1.0e6,
                     device="cuda", stream=None, out=None):
    """cos/sin table [max_position, rotary_dim] fp32 on the GPU (built by a HIP kernel)."""
    import torch
    lib = load_library()
    if out is None:
        out = torch.empty((max_position, rotary_dim), dtype=torch.float32, device=device)
    _check("pkv_rope_cache_build",
           lib.pkv_rope_cache_build(_ptr(out), max_position, rotary_dim, float(theta), _stream(stream)))
    return out


def qk_norm_rope(q, k, positions, q_norm_weight, k_norm_weight, cos_sin_cache, eps: float = 1.0e-6,
                 q_out=None, k_out=None, stream=None):
    """QK-Norm then RoPE.  q: [N, Hq, 128], k: [N, Hkv, 128] bf16 views (row-strided allowed).

    Returns (q_out, k_out), contiguous bf16.  Pass q_out=q / k_out=k to run in place
    on contiguous inputs.
    """
    import torch
    lib = load_library()
    n, hq, hkv = q.shape[0], q.shape[1], k.shape[1]
    qs, ks = _rows(q, hq, "q"), _rows(k, hkv, "k")
    if k.shape[0] != n or positions.shape[0] != n:
        raise ValueError("q, k and positions must have the same number of tokens")
    if positions.dtype != torch.int64 or not positions.is_contiguous():
        raise TypeError("positions must be a contiguous int64 tensor")
    _same_device(q, k=k, positions=positions)
    _norm_params(q_norm_weight, k_norm_weight, cos_sin_cache, q)
    if q_out is None:
        q_out = torch.empty((n, hq, HEAD_DIM), dtype=torch.bfloat16, device=q.device)
    if k_out is None:
        k_out = torch.empty((n, hkv, HEAD_DIM), dtype=torch.bfloat16, device=k.device)
    _out(q_out, (n, hq, HEAD_DIM), q, "q_out")
    _out(k_out, (n, hkv, HEAD_DIM), q, "k_out")
    _check("pkv_qk_norm_rope",
           lib.pkv_qk_norm_rope(_ptr(q), qs, _ptr(k), ks, _ptr(q_out), _ptr(k_out), _ptr(positions), n, hq, hkv,
                                HEAD_DIM, _ptr(q_norm_weight), _ptr(k_norm_weight), float(eps),
                                _ptr(cos_sin_cache), cos_sin_cache.shape[0], _stream(stream)))
    return q_out, k_out


def qk_norm_rope_store(q, k, v, positions, q_norm_weight, k_norm_weight, cos_sin_cache, k_cache, v_cache,
                       slot_mapping, eps: float = 1.0e-6, q_out=None, k_out=None, stream=None):
    """QK-Norm + RoPE with the cache scatter fused in.  q: [N, Hq, 128], k, v: [N, Hkv, 128]
    bf16 views (row-strided allowed); caches [num_blocks, 256, Hkv, 128]; slot_mapping [N] int32.

    The rotated keys and the values land in their cache rows; returns q_out (contiguous,
    allocated if not given; q_out=q runs in place).  k_out, if given, also receives the
    rotated keys.
    """
    import torch
    lib = load_library()
    n, hq, hkv = q.shape[0], q.shape[1], k.shape[1]
    qs, ks, vs = _rows(q, hq, "q"), _rows(k, hkv, "k"), _rows(v, hkv, "v")
    if k.shape[0] != n or v.shape[0] != n or positions.shape[0] != n or slot_mapping.numel() != n:
        raise ValueError("q, k, v, positions and slot_mapping must have the same number of tokens")
    if positions.dtype != torch.int64 or not positions.is_contiguous():
        raise TypeError("positions must be a contiguous int64 tensor")
    _i32(slot_mapping, "slot_mapping")
    D = hkv * HEAD_DIM
    for c in (k_cache, v_cache):
        if c.dtype != torch.bfloat16 or not c.is_contiguous() or c.dim() != 4 or c.stride(1) != D:
            raise ValueError("caches must be contiguous bf16 [num_blocks, block_size, Hkv, 128]")
    if k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache must have the same shape")
    _same_device(q, k=k, v=v, positions=positions, slot_mapping=slot_mapping, k_cache=k_cache, v_cache=v_cache)
    _norm_params(q_norm_weight, k_norm_weight, cos_sin_cache, q)
    if q_out is None:
        q_out = torch.empty((n, hq, HEAD_DIM), dtype=torch.bfloat16, device=q.device)
    _out(q_out, (n, hq, HEAD_DIM), q, "q_out")
    if k_out is not None:
        _out(k_out, (n, hkv, HEAD_DIM), q, "k_out")
    _check("pkv_qk_norm_rope_store",
           lib.pkv_qk_norm_rope_store(_ptr(q), qs, _ptr(k), ks, _ptr(v), vs, _ptr(q_out), _ptr(k_out),
                                      _ptr(k_cache), _ptr(v_cache), k_cache.numel() // D, _ptr(slot_mapping),
                                      _ptr(positions), n, hq, hkv, HEAD_DIM, _ptr(q_norm_weight),
                                      _ptr(k_norm_weight), float(eps), _ptr(cos_sin_cache),
                                      cos_sin_cache.shape[0], _stream(stream)))
    return q_out


def store_kvcache(key, value, k_cache, v_cache, slot_mapping, stream=None):
    """Scatter key/value rows [N, Hkv, 128] into the paged caches [num_blocks, 256, Hkv, 128]."""
    lib = load_library()
    n, hkv = key.shape[0], key.shape[1]
    ks, vs = _rows(key, hkv, "key"), _rows(value, hkv, "value")
    D = hkv * HEAD_DIM
    if k_cache.stride(1) != D or v_cache.stride(1) != D or not (k_cache.is_contiguous() and v_cache.is_contiguous()):
        raise ValueError("caches must be contiguous with stride(1) == num_kv_heads*head_dim")
    if slot_mapping.numel() != n or value.shape[0] != n or value.shape[1] != hkv:
        raise ValueError("key, value and slot_mapping must have the same number of tokens and heads")
    _i32(slot_mapping, "slot_mapping")
    if k_cache.dtype != key.dtype or v_cache.dtype != key.dtype or value.dtype != key.dtype or \
            k_cache.numel() != v_cache.numel():
        raise ValueError("key, value and both caches must share one dtype, and the caches one size")
    _same_device(key, value=value, k_cache=k_cache, v_cache=v_cache, slot_mapping=slot_mapping)
    num_slots = k_cache.numel() // D
    _check("pkv_store_kvcache",
           lib.pkv_store_kvcache(_ptr(key), ks, _ptr(value), vs, _ptr(k_cache), _ptr(v_cache), num_slots,
                                 _ptr(slot_mapping), n, hkv, HEAD_DIM, key.element_size(), _stream(stream)))


def prefill_workspace_bytes(num_seqs: int, total_q: int, max_seqlen_q: int, max_seqlen_k: int, num_q_heads: int,
                            num_kv_heads: int) -> int:
    """Bytes of the optional key-split workspace of a prefill call of these sizes (0: no split)."""
    return int(load_library().pkv_attn_prefill_workspace_bytes(num_seqs, total_q, int(max_seqlen_q),
                                                               int(max_seqlen_k), num_q_heads, num_kv_heads,
                                                               HEAD_DIM))


def attn_prefill_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int,
                        softmax_scale: Optional[float] = None, causal: bool = True, block_table=None, out=None,
                        workspace=None, stream=None):
    """Varlen causal GQA prefill.  q: [Tq, Hq, 128]; k/v: [Tk, Hkv, 128] (case 1) or the caches
    [num_blocks, 256, Hkv, 128] with block_table [B, max_blocks] (case 2).  Returns o [Tq, Hq, 128].
    workspace: a uint8 device tensor for the key split (None: allocated here when the call
    would split; an empty tensor: run unsplit)."""
    import torch
    lib = load_library()
    tq, hq = q.shape[0], q.shape[1]
    qs = _rows(q, hq, "q")
    if block_table is not None:
        if k.dim() != 4 or k.shape[1] != BLOCK_SIZE or not (k.is_contiguous() and v.is_contiguous()):
            raise ValueError("with block_table, k and v must be contiguous caches [num_blocks, 256, Hkv, 128]")
        hkv, num_blocks = k.shape[2], k.shape[0]
        ks = vs = hkv * HEAD_DIM
        _i32(block_table, "block_table")
        mb = block_table.shape[1]
    else:
        hkv = k.shape[1]
        ks, vs = _rows(k, hkv, "k"), _rows(v, hkv, "v")
        num_blocks, mb = 0, 0
    _i32(cu_seqlens_q, "cu_seqlens_q")
    _i32(cu_seqlens_k, "cu_seqlens_k")
    nseq = cu_seqlens_q.numel() - 1
    if cu_seqlens_k.numel() != nseq + 1:
        raise ValueError(f"cu_seqlens_k must hold num_seqs + 1 = {nseq + 1} entries, got {cu_seqlens_k.numel()}")
    if block_table is not None and (block_table.dim() != 2 or block_table.shape[0] < nseq):
        raise ValueError(f"block_table must be [num_seqs >= {nseq}, max_blocks], got {tuple(block_table.shape)}")
    if k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16 or (block_table is not None and k.shape != v.shape):
        raise ValueError("k and v must be bfloat16 (and, as caches, of the same shape)")
    _same_device(q, k=k, v=v, cu_seqlens_q=cu_seqlens_q, cu_seqlens_k=cu_seqlens_k, block_table=block_table)
    scale = HEAD_DIM ** -0.5 if softmax_scale is None else softmax_scale
    if out is None:
        out = torch.empty((tq, hq, HEAD_DIM), dtype=torch.bfloat16, device=q.device)
    _out(out, (tq, hq, HEAD_DIM), q, "out")
    if workspace is None:
        need = prefill_workspace_bytes(nseq, tq, max_seqlen_q, max_seqlen_k, hq, hkv)
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device) if need else None
    elif workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor")
    else:
        _same_device(q, workspace=workspace)
    ws_ptr, ws_bytes = (_ptr(workspace), workspace.numel()) if workspace is not None and workspace.numel() else (None, 0)
    _check("pkv_attn_prefill_varlen",
           lib.pkv_attn_prefill_varlen(_ptr(q), qs, _ptr(k), ks, _ptr(v), vs, _ptr(out), _ptr(cu_seqlens_q),
                                       _ptr(cu_seqlens_k), nseq, tq, int(max_seqlen_q), int(max_seqlen_k), hq, hkv,
                                       HEAD_DIM, float(scale), 1 if causal else 0, _ptr(block_table), mb,
                                       BLOCK_SIZE, num_blocks, ws_ptr, ws_bytes, _stream(stream)))
    return out


def decode_workspace_bytes(num_seqs: int, num_q_heads: int, num_kv_heads: int, max_blocks_per_seq: int) -> int:
    lib = load_library()
    return int(lib.pkv_attn_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, HEAD_DIM,
                                                   max_blocks_per_seq, BLOCK_SIZE))


def attn_decode_paged(q, k_cache, v_cache, cache_seqlens, block_table, softmax_scale: Optional[float] = None,
                      causal: bool = True, out=None, workspace=None, stream=None):
    """Paged decode.  q: [B, Hq, 128] (or [B, 1, Hq, 128]); caches [num_blocks, 256, Hkv, 128];
    cache_seqlens [B] int32 (tokens in cache, the new one included); block_table [B, max_blocks]."""
    import torch
    lib = load_library()
    if q.dim() == 4:
        if q.shape[1] != 1:
            raise ValueError("decode takes exactly one query per sequence")
        q = q[:, 0]
    if not q.is_contiguous():
        raise ValueError("q must be contiguous [B, Hq, 128]")
    B, hq = q.shape[0], q.shape[1]
    _rows(q, hq, "q")
    if k_cache.dim() != 4 or k_cache.shape[1] != BLOCK_SIZE or not (k_cache.is_contiguous() and v_cache.is_contiguous()):
        raise ValueError("caches must be contiguous [num_blocks, 256, Hkv, 128]")
    hkv, num_blocks = k_cache.shape[2], k_cache.shape[0]
    _i32(cache_seqlens, "cache_seqlens")
    _i32(block_table, "block_table")
    if cache_seqlens.numel() != B or block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError(f"cache_seqlens [B] and block_table [B, max_blocks] must match q's B = {B}, got "
                         f"{tuple(cache_seqlens.shape)} and {tuple(block_table.shape)}")
    if k_cache.dtype != torch.bfloat16 or k_cache.shape != v_cache.shape:
        raise ValueError("caches must be bfloat16 and of the same shape")
    _same_device(q, k_cache=k_cache, v_cache=v_cache, cache_seqlens=cache_seqlens, block_table=block_table,
                 workspace=workspace)
    mb = block_table.shape[1]
    scale = HEAD_DIM ** -0.5 if softmax_scale is None else softmax_scale
    need = decode_workspace_bytes(B, hq, hkv, mb)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    if workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor")
    if out is None:
        out = torch.empty((B, hq, HEAD_DIM), dtype=torch.bfloat16, device=q.device)
    _out(out, (B, hq, HEAD_DIM), q, "out")
    _check("pkv_attn_decode_paged",
           lib.pkv_attn_decode_paged(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(cache_seqlens),
                                     _ptr(block_table), mb, B, hq, hkv, HEAD_DIM, BLOCK_SIZE, num_blocks,
                                     float(scale), _ptr(workspace), workspace.numel(), _stream(stream)))
    return out


def add_rms_norm(x, residual, weight, eps: float = 1.0e-6, y=None, residual_out=None, stream=None):
    """RMSNorm of x + residual over the last dim (bf16 [T, hidden], contiguous).

    Returns (y, new_residual).  With residual None, plain RMSNorm of x: returns (y, x).
    Pass y=x / residual_out=residual to run in place."""
    import torch
    lib = load_library()
    if x.dtype != torch.bfloat16 or x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous bf16 [T, hidden] tensor")
    t, hidden = x.shape
    if residual is not None and (residual.shape != x.shape or residual.dtype != x.dtype or
                                 not residual.is_contiguous()):
        raise ValueError("residual must match x")
    if weight.dtype != torch.bfloat16 or weight.numel() != hidden or not weight.is_contiguous():
        raise ValueError(f"weight must be a contiguous bfloat16 tensor of {hidden} elements")
    _same_device(x, residual=residual, weight=weight)
    if y is None:
        y = torch.empty_like(x)
    if residual is not None and residual_out is None:
        residual_out = torch.empty_like(x)
    _out(y, x.shape, x, "y")
    if residual is not None:
        _out(residual_out, x.shape, x, "residual_out")
    _check("pkv_add_rms_norm",
           lib.pkv_add_rms_norm(_ptr(x), _ptr(residual), _ptr(weight), _ptr(y),
                                _ptr(residual_out) if residual is not None else None, t, hidden, float(eps),
                                _stream(stream)))
    return y, (residual_out if residual is not None else x)


def silu_and_mul(x, out=None, stream=None):
    """x bf16 [T, 2I] (gate | up) -> silu(gate) * up, bf16 [T, I]."""
    import torch
    lib = load_library()
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a bf16 [T, 2I] tensor with unit column stride")
    t, two_i = x.shape
    if two_i % 2:
        raise ValueError("x must hold gate and up halves of equal width")
    inter = two_i // 2
    if out is None:
        out = torch.empty((t, inter), dtype=torch.bfloat16, device=x.device)
    if out.dtype != torch.bfloat16 or tuple(out.shape) != (t, inter) or out.stride(1) != 1 or out.device != x.device:
        raise ValueError(f"out must be a bfloat16 [{t}, {inter}] tensor with unit column stride on {x.device}")
    _check("pkv_silu_and_mul",
           lib.pkv_silu_and_mul(_ptr(x), x.stride(0), _ptr(out), out.stride(0), t, inter, _stream(stream)))
    return out


def sample_gumbel(logits, temperatures, seed: int = 0, offset: int = 0, noise=None, out=None, stream=None):
    """One token per row: argmax softmax(logits / T) / E, E ~ Exp(1) (in-kernel Philox unless
    ``noise`` [B, V] fp32 is given).  logits bf16 or fp32 [B, V]; returns int64 [B]."""
    import torch
    lib = load_library()
    if logits.dim() != 2 or logits.stride(1) != 1:
        raise ValueError("logits must be [B, V] with unit column stride")
    dt = {torch.bfloat16: 0, torch.float32: 1}.get(logits.dtype)
    if dt is None:
        raise TypeError("logits must be bfloat16 or float32")
    b, v = logits.shape
    if temperatures.dtype != torch.float32 or temperatures.numel() != b or not temperatures.is_contiguous():
        raise ValueError("temperatures must be contiguous float32 [B]")
    if noise is not None and (noise.dtype != torch.float32 or noise.shape != logits.shape or noise.stride(1) != 1):
        raise ValueError("noise must be float32 [B, V]")
    _same_device(logits, temperatures=temperatures, noise=noise)
    if out is None:
        out = torch.empty(b, dtype=torch.int64, device=logits.device)
    if out.dtype != torch.int64 or out.numel() != b or not out.is_contiguous() or out.device != logits.device:
        raise ValueError(f"out must be a contiguous int64 tensor of {b} elements on {logits.device}")
    _check("pkv_sample_gumbel",
           lib.pkv_sample_gumbel(_ptr(logits), logits.stride(0), dt, _ptr(temperatures), _ptr(noise),
                                 noise.stride(0) if noise is not None else 0, int(seed), int(offset), _ptr(out), b, v,
                                 _stream(stream)))
    return out


class DecodeStep:
    """The decode step over static buffers sized for ``max_batch`` rows.

    ``qkv`` [max_batch, W] bf16 holds the step's q | k | v columns; ``positions``
    (int64), ``slot_mapping`` and ``context_lens`` (int32) [max_batch] and
    ``block_table`` [max_batch, max_blocks] are written by the caller before
    each step.  ``run(batch)`` launches the kernels eagerly; ``capture()``
    records one HIP graph per bucket and ``replay(batch)`` pads rows
    [batch, bucket) (slot -1, context 0) and launches the bucket's graph.
    With ``caller_pads=True`` the caller keeps those rows padded itself and a
    replay launches the graph alone.
    Outputs: ``q_out`` (q') and ``o`` [max_batch, Hq, 128].
    """

    def __init__(self, qkv, k_cache, v_cache, positions, slot_mapping, context_lens, block_table, q_norm_weight,
                 k_norm_weight, cos_sin_cache, num_q_heads: int, num_kv_heads: int, eps: float = 1.0e-6,
                 softmax_scale: Optional[float] = None, caller_pads: bool = False):
        import torch
        lib = load_library()
        mb = qkv.shape[0]
        if qkv.dtype != torch.bfloat16 or qkv.dim() != 2 or qkv.stride(1) != 1:
            raise ValueError("qkv must be a bf16 [max_batch, W] tensor with unit column stride")
        for t, name in ((positions, "positions"), (slot_mapping, "slot_mapping"), (context_lens, "context_lens"),
                        (block_table, "block_table")):
            if t.shape[0] != mb or not t.is_contiguous():
                raise ValueError(f"{name} must be contiguous with max_batch = {mb} rows")
        if positions.dtype != torch.int64:
            raise TypeError("positions must be int64")
        _i32(slot_mapping, "slot_mapping")
        _i32(context_lens, "context_lens")
        _i32(block_table, "block_table")
        if k_cache.dim() != 4 or k_cache.shape[1] != BLOCK_SIZE or not (k_cache.is_contiguous() and
                                                                        v_cache.is_contiguous()):
            raise ValueError("caches must be contiguous [num_blocks, 256, Hkv, 128]")
        self.q_out = torch.empty((mb, num_q_heads, HEAD_DIM), dtype=torch.bfloat16, device=qkv.device)
        self.o = torch.empty_like(self.q_out)
        need = int(lib.pkv_decode_step_workspace_bytes(mb, num_q_heads, num_kv_heads, HEAD_DIM, block_table.shape[1],
                                                       BLOCK_SIZE))
        if need == 0:
            raise ValueError("invalid decode sizes")
        self.workspace = torch.empty(need, dtype=torch.uint8, device=qkv.device)
        self._keep = (qkv, k_cache, v_cache, positions, slot_mapping, context_lens, block_table, q_norm_weight,
                      k_norm_weight, cos_sin_cache)
        self.max_batch = mb
        self.desc = DecodeStepDesc(
            qkv=_ptr(qkv), qkv_row_stride=qkv.stride(0), q_out=_ptr(self.q_out), o=_ptr(self.o),
            k_cache=_ptr(k_cache), v_cache=_ptr(v_cache), num_blocks=k_cache.shape[0], positions=_ptr(positions),
            slot_mapping=_ptr(slot_mapping), context_lens=_ptr(context_lens), block_table=_ptr(block_table),
            max_blocks_per_seq=block_table.shape[1], max_batch=mb, q_norm_weight=_ptr(q_norm_weight),
            k_norm_weight=_ptr(k_norm_weight), cos_sin_cache=_ptr(cos_sin_cache),
            max_position=cos_sin_cache.shape[0], eps=float(eps), num_q_heads=num_q_heads,
            num_kv_heads=num_kv_heads, head_dim=HEAD_DIM, block_size=BLOCK_SIZE,
            softmax_scale=HEAD_DIM ** -0.5 if softmax_scale is None else float(softmax_scale),
            flags=PKV_DECODE_CALLER_PADS if caller_pads else 0,
            workspace=_ptr(self.workspace), workspace_bytes=need)
        self._graph = None
        self.buckets = ()

    def run(self, batch: int, stream=None):
        """One eager step over rows 0..batch-1."""
        _check("pkv_decode_step", _lib.pkv_decode_step(ctypes.byref(self.desc), int(batch), _stream(stream)))

    def capture(self, buckets=None):
        """Capture one graph per bucket (default: the ladder up to max_batch)."""
        if buckets is None:
            buckets = [b for b in GRAPH_BUCKETS if b <= self.max_batch]
        self.close()
        arr = (ctypes.c_int32 * len(buckets))(*buckets)
        h = ctypes.c_void_p()
        _check("pkv_decode_graph_create",
               _lib.pkv_decode_graph_create(ctypes.byref(self.desc), arr, len(buckets), ctypes.byref(h)))
        self._graph = h
        self.buckets = tuple(int(b) for b in buckets)

    def bucket(self, batch: int) -> int:
        return int(_lib.pkv_decode_graph_bucket(self._graph, int(batch))) if self._graph else -1

    def replay(self, batch: int, stream=None):
        """One step over rows 0..batch-1 from the captured graph of its bucket."""
        if self._graph is None:
            raise RuntimeError("capture() first")
        _check("pkv_decode_graph_launch", _lib.pkv_decode_graph_launch(self._graph, int(batch), _stream(stream)))

    def close(self):
        if self._graph is not None:
            _lib.pkv_decode_graph_destroy(self._graph)
            self._graph = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
