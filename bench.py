"""Benchmark of the Qwen3-8B-shaped attention-sublayer core on one MI355X.

One step = one pass of the whole hot path over both 8B workloads:
  prefill phase  (16 sequences x 4096 tokens, first 2048 cached in shared blocks):
      qk_norm_rope over 32768 new tokens -> store_kvcache of their K/V ->
      paged causal prefill (2048 queries per sequence over 4096 keys);
  decode phase   (256 sequences, contexts log-uniform in [1024, 32768], 64 of them
                  sharing an 8-block prefix):
      qk_norm_rope over 256 tokens -> store_kvcache -> paged decode.

Inputs are synthetic and seeded (``workloads``), resident in HBM before timing.
Prints one JSON line.  ``value`` is the paged-decode attention throughput in GB/s
of algorithmic bytes (unique K/V bytes + q/o + metadata) over the decode call's
average duration; the causal-prefill TFLOP/s is reported beside it.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
METRIC = "paged decode attn HBM GB/s + causal prefill attn TFLOP/s, Qwen3-8B shapes, 1 GPU"


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def recorded_traffic(profile_name: str, source: str):
    """HBM bytes per launch recorded under profiles/ by rocprofv3 FETCH_SIZE/WRITE_SIZE runs.

    Returned only while the kernel source still hashes to what the profile recorded;
    a changed kernel reports null until it is profiled again.
    """
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", profile_name)
    src = os.path.join(ROOT, "paged_kv_gqa_amd", "csrc", source)
    if not (os.path.exists(path) and os.path.exists(src)):
        return None
    text = open(path).read()
    m_sha = re.search(r"source_sha256:\s*([0-9a-f]{64})", text)
    m_val = re.search(r"traffic_bytes_per_launch:\s*([0-9]+)", text)
    if not (m_sha and m_val):
        return None
    if hashlib.sha256(open(src, "rb").read()).hexdigest() != m_sha.group(1):
        return None
    return int(m_val.group(1))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seqs", type=int, default=24, help="decode sequences the oracle times")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run a plain 1 GiB device copy (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import paged_kv_gqa_amd as pkv
    import workloads as wl

    assert torch.cuda.is_available(), "bench needs a GPU"
    pkv.load_library()
    dev = torch.device("cuda:0")
    D = 128

    def to_dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    if args.calibrate_copy:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            t0 = time.perf_counter()
            dst.copy_(src)
            torch.cuda.synchronize()
            dt = time.perf_counter() - t0
        log(f"calibration copy: {src.numel() * 4 / 2**30:.0f} GiB read + written, {2 * src.numel() * 4 / dt / 1e9:.0f} GB/s")
        del src, dst

    # ---------------- set-up (untimed) ----------------
    s8 = wl.QWEN3_8B
    q0, k0, v0 = wl.qkv_views(s8)
    table = pkv.rope_cache_build(s8.max_position, D, s8.rope_theta, device=dev)

    wp = wl.prefix_prefill_8b(seed=args.seed)
    log(f"prefill workload: {wp.num_seqs} x {wp.total_len} tokens, {wp.num_q_tokens} queried, "
        f"{wp.num_blocks} blocks, {wp.flops / 1e12:.3f} TFLOP")
    Tq = wp.num_q_tokens
    qkv_p = torch.empty((Tq, s8.qkv_width), dtype=torch.bfloat16, device=dev)
    wl.fill_normal_bf16_(qkv_p, 5, args.seed, 1)
    gq_p, gk_p = (to_dev(g) for g in wp.gammas())
    kc_p = torch.empty((wp.num_blocks, 256, s8.num_kv_heads, D), dtype=torch.bfloat16, device=dev)
    vc_p = torch.empty_like(kc_p)
    wl.fill_normal_bf16_(kc_p, 5, args.seed, 10)
    wl.fill_normal_bf16_(vc_p, 5, args.seed, 11)
    pos_p, slot_p = to_dev(wp.positions), to_dev(wp.slot_mapping)
    cuq_p, cuk_p, bt_p = to_dev(wp.cu_seqlens_q), to_dev(wp.cu_seqlens_k), to_dev(wp.block_tables)
    qo_p = torch.empty((Tq, s8.num_q_heads, D), dtype=torch.bfloat16, device=dev)
    ko_p = torch.empty((Tq, s8.num_kv_heads, D), dtype=torch.bfloat16, device=dev)
    o_p = torch.empty((Tq, s8.num_q_heads, D), dtype=torch.bfloat16, device=dev)

    wd = wl.paged_decode_8b(seed=args.seed)
    B = wd.batch
    log(f"decode workload: {B} sequences, mean context {wd.context_lens.mean():.0f}, {wd.num_blocks} blocks, "
        f"{wd.algorithmic_bytes() / 1e9:.3f} GB unique ({wd.algorithmic_bytes(False) / 1e9:.3f} GB logical)")
    kc_d = torch.empty((wd.num_blocks, 256, s8.num_kv_heads, D), dtype=torch.bfloat16, device=dev)
    vc_d = torch.empty_like(kc_d)
    wl.fill_normal_bf16_(kc_d, 4, args.seed, 10)
    wl.fill_normal_bf16_(vc_d, 4, args.seed, 11)
    qkv_d = to_dev(wd.qkv())
    gq_d, gk_d = (to_dev(g) for g in wd.gammas())
    pos_d, slot_d = to_dev(wd.positions), to_dev(wd.slot_mapping)
    cl_d, bt_d = to_dev(wd.context_lens), to_dev(wd.block_tables)
    qo_d = torch.empty((B, s8.num_q_heads, D), dtype=torch.bfloat16, device=dev)
    ko_d = torch.empty((B, s8.num_kv_heads, D), dtype=torch.bfloat16, device=dev)
    o_d = torch.empty((B, s8.num_q_heads, D), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(pkv.decode_workspace_bytes(B, s8.num_q_heads, s8.num_kv_heads, wd.block_tables.shape[1]),
                     dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    qv_p = qkv_p[:, q0:k0].view(Tq, s8.num_q_heads, D)
    kv_p = qkv_p[:, k0:v0].view(Tq, s8.num_kv_heads, D)
    vv_p = qkv_p[:, v0:].view(Tq, s8.num_kv_heads, D)
    qv_d = qkv_d[:, q0:k0].view(B, s8.num_q_heads, D)
    kv_d = qkv_d[:, k0:v0].view(B, s8.num_kv_heads, D)
    vv_d = qkv_d[:, v0:].view(B, s8.num_kv_heads, D)
    stream = torch.cuda.current_stream()
    names = ["norm_rope_p", "store_p", "prefill", "norm_rope_d", "store_d", "decode"]

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record(stream)
        mark(0)
        pkv.qk_norm_rope(qv_p, kv_p, pos_p, gq_p, gk_p, table, s8.eps, q_out=qo_p, k_out=ko_p)
        mark(1)
        pkv.store_kvcache(ko_p, vv_p, kc_p, vc_p, slot_p)
        mark(2)
        pkv.attn_prefill_varlen(qo_p, kc_p, vc_p, cuq_p, cuk_p, wp.suffix_len, wp.total_len, block_table=bt_p,
                                out=o_p)
        mark(3)
        pkv.qk_norm_rope(qv_d, kv_d, pos_d, gq_d, gk_d, table, s8.eps, q_out=qo_d, k_out=ko_d)
        mark(4)
        pkv.store_kvcache(ko_d, vv_d, kc_d, vc_d, slot_d)
        mark(5)
        pkv.attn_decode_paged(qo_d, kc_d, vc_d, cl_d, bt_d, out=o_d, workspace=ws)
        mark(6)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(args.steps)]
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = {n: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in events])) for j, n in enumerate(names)}
    ms_step = wall * 1e3 / args.steps

    dec_bytes = wd.algorithmic_bytes(unique=True)
    dec_gbs = dec_bytes / (per["decode"] * 1e-3) / 1e9
    pre_tflops = wp.flops / (per["prefill"] * 1e-3) / 1e12
    store_bytes = wp.store_bytes
    norm_bytes = Tq * ((s8.num_q_heads + s8.num_kv_heads) * D * 2 * 2 + 8 + 512)
    kernels = {
        "attn_decode_paged": {"ms": per["decode"], "GB/s": dec_gbs, "bytes": dec_bytes,
                              "logical_bytes": wd.algorithmic_bytes(unique=False)},
        "attn_prefill_varlen": {"ms": per["prefill"], "TFLOP/s": pre_tflops, "flop": wp.flops},
        "store_kvcache_prefill": {"ms": per["store_p"], "GB/s": store_bytes / (per["store_p"] * 1e-3) / 1e9,
                                  "bytes": store_bytes},
        "qk_norm_rope_prefill": {"ms": per["norm_rope_p"], "GB/s": norm_bytes / (per["norm_rope_p"] * 1e-3) / 1e9,
                                 "bytes": norm_bytes},
        "qk_norm_rope_decode": {"ms": per["norm_rope_d"]},
        "store_kvcache_decode": {"ms": per["store_d"]},
    }
    log(json.dumps(kernels))

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args, wd, kc_d, vc_d, qo_d, log)

    out = {
        "metric": METRIC,
        "value": round(dec_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "qwen3-8b attention core: paged decode (256 seqs, ctx log-U[1024,32768], 64 share an "
                        "8-block prefix) + prefix-hit causal prefill (16 x 4096 tokens, 2048 cached)",
            "num_q_heads": 32, "num_kv_heads": 8, "head_dim": 128, "block_size": 256,
            "decode_batch": B, "prefill_seqs": wp.num_seqs, "prefill_query_tokens": Tq, "parallelism": "none",
        },
        "prefill": {"value": round(pre_tflops, 2), "unit": "TFLOP/s", "ms": round(per["prefill"], 4)},
        "roofline": {"bound": "hbm", "kernel": "attn_decode_paged", "achieved": round(dec_gbs, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic("attn_decode_paged_qwen3_8b_hbm_traffic.md", "attn_decode.hip")},
        "roofline_prefill": {"bound": "mfma", "kernel": "attn_prefill_varlen", "achieved": round(pre_tflops, 2),
                             "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                             "frac": round(pre_tflops / BF16_PEAK_TFLOPS, 4),
                             "traffic": recorded_traffic("attn_prefill_qwen3_8b_prefix_hbm_traffic.md",
                                                         "attn_prefill.hip")},
        "kernels": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                    for k, v in kernels.items()},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def cpu_baseline(args, wd, kc_d, vc_d, q_d, log):
    """The oracle's paged decode on a bounded sample of the same workload, on the host cores."""
    import torch

    import oracle
    import workloads as wl

    def bits(t):
        return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    def gather_sequences(k_cache, v_cache, block_table, seqs, context_lens):
        rows = [[int(x) for x in block_table[b, :-(-int(context_lens[b]) // 256)]] for b in seqs]
        uniq = sorted({p for r in rows for p in r})
        where = {p: i for i, p in enumerate(uniq)}
        idx = torch.tensor(uniq, dtype=torch.int64, device=k_cache.device)
        hkv = k_cache.shape[2]
        kc = bits(k_cache.index_select(0, idx)).reshape(len(uniq) * 256, hkv, 128)
        vc = bits(v_cache.index_select(0, idx)).reshape(len(uniq) * 256, hkv, 128)
        return kc, vc, wl.pad_block_tables([[where[p] for p in r] for r in rows], block_table.shape[1])

    rng = np.random.default_rng(args.seed + 100)
    seqs = sorted(rng.choice(wd.batch, size=min(args.cpu_seqs, wd.batch), replace=False).tolist())
    kc, vc, bt = gather_sequences(kc_d, vc_d, wd.block_tables, seqs, wd.context_lens)
    q = bits(q_d)[seqs]
    cl = wd.context_lens[seqs]
    oracle.attn_decode(q[:1], kc, vc, cl[:1], bt[:1], 32, 8)       # warm the library
    t0 = time.perf_counter()
    oracle.attn_decode(q, kc, vc, cl, bt, 32, 8)
    dt = time.perf_counter() - t0
    nbytes = int(np.sum(cl.astype(np.int64))) * 8 * 128 * 2 * 2 + len(seqs) * 32 * 128 * 2 * 2
    log(f"cpu baseline: {len(seqs)} sequences, {nbytes / 1e9:.3f} GB in {dt:.2f} s")
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"paged decode of {len(seqs)} of the {wd.batch} sequences ({int(np.sum(cl))} context tokens, "
                      f"32 q heads), fp64 C oracle with OpenMP, {dt:.2f} s"}


if __name__ == "__main__":
    main()
