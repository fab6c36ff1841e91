"""Benchmark of the Qwen3-8B-shaped attention-sublayer core on one MI355X.

One step = one pass of the whole hot path over both 8B workloads:
  prefill phase  (16 sequences x 4096 tokens, first 2048 cached in shared blocks):
      QK-Norm + RoPE over 32768 new tokens with their K/V scattered into the
      cache in the same pass -> paged causal prefill (2048 queries per sequence
      over 4096 keys);
  decode phase   (256 sequences, contexts log-uniform in [1024, 32768], 64 of them
                  sharing an 8-block prefix):
      QK-Norm + RoPE + scatter of the 256 new tokens -> paged decode.
The unfused pair (qk_norm_rope, then store_kvcache) is timed separately after
the step loop and reported under "kernels".

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


def gpu_lead(torch, ms: float):
    """Keep the GPU busy for about `ms` milliseconds (a spin kernel) so that the host
    enqueues the calls that follow before the GPU reaches them: the events around a
    batch of short calls then time the kernels, not the host's launch work between them."""
    try:
        torch.cuda._sleep(int(ms * 2.5e6))   # cycles; at most 2.5 GHz, so at least `ms`
    except (AttributeError, RuntimeError):
        pass


def input_checksum(torch, named):
    """sha256 (first 16 hex digits) over each input's name, shape, dtype, the sum of its
    32-bit words and their position-weighted sum (word i times (i * 2654435761) mod 2^32,
    int64 arithmetic wrapping mod 2^64; device reduction in 16M-word pieces).  Recorded with
    the seed so a run's synthetic inputs can be told apart from another's; the weighted sum
    also tells a permuted block table or slot map from the original."""
    import hashlib
    h = hashlib.sha256()
    for name, t in named:
        flat = t.reshape(-1).view(torch.int32) if t.element_size() * t.numel() % 4 == 0 else t.reshape(-1)
        total = weighted = 0
        step = 1 << 24
        for i in range(0, flat.numel(), step):
            piece = flat[i:i + step].to(torch.int64)
            idx = torch.arange(i, i + piece.numel(), dtype=torch.int64, device=piece.device)
            w = (idx * 2654435761) & 0xFFFFFFFF
            total += int(torch.sum(piece).item())
            weighted = (weighted + int(torch.sum(piece * w).item())) % (1 << 64)
        h.update(f"{name}:{tuple(t.shape)}:{t.dtype}:{total}:{weighted};".encode())
    return h.hexdigest()[:16]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ladders", action="store_true",
                    help="skip the decode-step graph measurements (ladders and the layer stack), as the "
                         "counter runs behind profiles/ do")
    ap.add_argument("--cpu-seqs", type=int, default=256, help="decode sequences the oracle times")
    ap.add_argument("--cpu-prefill-rows", type=int, default=131072, help="prefill (token, head) rows the oracle times")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run a plain 1 GiB device copy (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this library has no multi-GPU path (asked for --gpus {args.gpus})",
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

    checksum = input_checksum(torch, [
        ("prefill.qkv", qkv_p), ("prefill.k_cache", kc_p), ("prefill.v_cache", vc_p), ("prefill.positions", pos_p),
        ("prefill.slot_mapping", slot_p), ("prefill.cu_seqlens_q", cuq_p), ("prefill.cu_seqlens_k", cuk_p),
        ("prefill.block_tables", bt_p), ("decode.qkv", qkv_d), ("decode.k_cache", kc_d), ("decode.v_cache", vc_d),
        ("decode.positions", pos_d), ("decode.slot_mapping", slot_d), ("decode.context_lens", cl_d),
        ("decode.block_tables", bt_d)])
    log(f"inputs: seed {args.seed}, checksum {checksum}")
    qv_p = qkv_p[:, q0:k0].view(Tq, s8.num_q_heads, D)
    kv_p = qkv_p[:, k0:v0].view(Tq, s8.num_kv_heads, D)
    vv_p = qkv_p[:, v0:].view(Tq, s8.num_kv_heads, D)
    qv_d = qkv_d[:, q0:k0].view(B, s8.num_q_heads, D)
    kv_d = qkv_d[:, k0:v0].view(B, s8.num_kv_heads, D)
    vv_d = qkv_d[:, v0:].view(B, s8.num_kv_heads, D)
    stream = torch.cuda.current_stream()
    names = ["norm_rope_store_p", "prefill", "norm_rope_store_d", "decode"]

    def step(ev=None):
        """QK-Norm + RoPE + cache scatter (one fused pass) then attention, for both phases."""
        def mark(i):
            if ev is not None:
                ev[i].record(stream)
        mark(0)
        pkv.qk_norm_rope_store(qv_p, kv_p, vv_p, pos_p, gq_p, gk_p, table, kc_p, vc_p, slot_p, s8.eps, q_out=qo_p)
        mark(1)
        pkv.attn_prefill_varlen(qo_p, kc_p, vc_p, cuq_p, cuk_p, wp.suffix_len, wp.total_len, block_table=bt_p,
                                out=o_p)
        mark(2)
        pkv.qk_norm_rope_store(qv_d, kv_d, vv_d, pos_d, gq_d, gk_d, table, kc_d, vc_d, slot_d, s8.eps, q_out=qo_d)
        mark(3)
        pkv.attn_decode_paged(qo_d, kc_d, vc_d, cl_d, bt_d, out=o_d, workspace=ws)
        mark(4)

    unfused_names = ["norm_rope_p", "store_p", "norm_rope_d", "store_d"]

    def unfused(ev):
        """The same first steps as two separate calls each (QK-Norm + RoPE, then the scatter)."""
        ev[0].record(stream)
        pkv.qk_norm_rope(qv_p, kv_p, pos_p, gq_p, gk_p, table, s8.eps, q_out=qo_p, k_out=ko_p)
        ev[1].record(stream)
        pkv.store_kvcache(ko_p, vv_p, kc_p, vc_p, slot_p)
        ev[2].record(stream)
        pkv.qk_norm_rope(qv_d, kv_d, pos_d, gq_d, gk_d, table, s8.eps, q_out=qo_d, k_out=ko_d)
        ev[3].record(stream)
        pkv.store_kvcache(ko_d, vv_d, kc_d, vc_d, slot_d)
        ev[4].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(args.steps)]
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = {n: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in events])) for j, n in enumerate(names)}
    spread = {n: (float(np.median([e[j].elapsed_time(e[j + 1]) for e in events])),
                  float(np.min([e[j].elapsed_time(e[j + 1]) for e in events]))) for j, n in enumerate(names)}
    ms_step = wall * 1e3 / args.steps

    # the unfused first steps, timed after the step loop (not part of ms_per_step)
    for _ in range(args.warmup):
        unfused([torch.cuda.Event(enable_timing=True) for _ in range(5)])
    uev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    gpu_lead(torch, 2.0 * args.steps)
    for i in range(args.steps):
        unfused(uev[i])
    torch.cuda.synchronize()
    per.update({n: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in uev])) for j, n in enumerate(unfused_names)})

    dec_bytes = wd.algorithmic_bytes(unique=True)
    dec_gbs = dec_bytes / (per["decode"] * 1e-3) / 1e9
    pre_tflops = wp.flops / (per["prefill"] * 1e-3) / 1e12
    store_bytes = wp.store_bytes
    hq8, hkv8 = s8.num_q_heads, s8.num_kv_heads
    # per token: q, k read + q', k' written; positions (8 B) and one table row (512 B) read
    norm_bytes = Tq * ((hq8 + hkv8) * D * 2 * 2 + 8 + 512)
    # fused, per token: q, k, v read + q', k', v written; position, slot id and table row read
    fused_bytes = Tq * ((hq8 + 2 * hkv8) * D * 2 * 2 + 8 + 4 + 512)

    def gbs(nbytes, ms):
        return nbytes / (ms * 1e-3) / 1e9

    kernels = {
        "attn_decode_paged": {"ms": per["decode"], "ms_median": spread["decode"][0], "ms_min": spread["decode"][1],
                              "GB/s": dec_gbs, "bytes": dec_bytes,
                              "logical_bytes": wd.algorithmic_bytes(unique=False)},
        "attn_prefill_varlen": {"ms": per["prefill"], "ms_median": spread["prefill"][0],
                                "ms_min": spread["prefill"][1], "TFLOP/s": pre_tflops, "flop": wp.flops},
        "qk_norm_rope_store_prefill": {"ms": per["norm_rope_store_p"],
                                       "GB/s": gbs(fused_bytes, per["norm_rope_store_p"]), "bytes": fused_bytes},
        "qk_norm_rope_store_decode": {"ms": per["norm_rope_store_d"]},
        "unfused_store_kvcache_prefill": {"ms": per["store_p"], "GB/s": gbs(store_bytes, per["store_p"]),
                                          "bytes": store_bytes},
        "unfused_qk_norm_rope_prefill": {"ms": per["norm_rope_p"], "GB/s": gbs(norm_bytes, per["norm_rope_p"]),
                                         "bytes": norm_bytes},
        "unfused_qk_norm_rope_decode": {"ms": per["norm_rope_d"]},
        "unfused_store_kvcache_decode": {"ms": per["store_d"]},
    }
    log(json.dumps(kernels))

    ops = sublayer_ops(pkv, torch, dev, to_dev, args, log)
    norm_small = norm_rope_small(pkv, torch, dev, table, args, log)
    small = qwen3_0_6b_shapes(pkv, torch, dev, to_dev, args, log)
    copy_ref = copy_reference(torch, dev, log)

    ladder = ladder_short = stack = None
    if not args.no_ladders:
        ladder = decode_graph_ladder(pkv, torch, s8, table, qkv_d, kc_d, vc_d, pos_d, slot_d, cl_d, bt_d, gq_d, gk_d,
                                     args, log)
        ladder_short = decode_graph_short(pkv, torch, dev, to_dev, table, args, log)
        stack = decode_graph_stack(pkv, torch, dev, to_dev, table, args, log)

    cpu = cpu_pre = cpu_st = cpu_one = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args, wd, kc_d, vc_d, qo_d, o_d, log)
        cpu_pre = cpu_baseline_prefill(args, wp, kc_p, vc_p, qo_p, o_p, log)
        cpu_st = cpu_stages(args, wp, qkv_p, log)
        cpu_one = cpu_one_thread(args, log)

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
        "inputs": {"seed": args.seed, "checksum": checksum},
        "config": {
            "workload": "qwen3-8b attention core: paged decode (256 seqs, ctx log-U[1024,32768], 64 share an "
                        "8-block prefix) + prefix-hit causal prefill (16 x 4096 tokens, 2048 cached)",
            "num_q_heads": 32, "num_kv_heads": 8, "head_dim": 128, "block_size": 256,
            "decode_batch": B, "prefill_seqs": wp.num_seqs, "prefill_query_tokens": Tq, "parallelism": "none",
        },
        "prefill": {"value": round(pre_tflops, 2), "unit": "TFLOP/s", "ms": round(per["prefill"], 4)},
        "roofline": {"bound": "hbm", "kernel": "attn_decode_paged", "achieved": round(dec_gbs, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic("attn_decode_paged_qwen3_8b_hbm_traffic.md", "attn_decode.hip"),
                     "measured_copy_GB/s": copy_ref["copy_GB/s"]},
        "roofline_prefill": {"bound": "mfma", "kernel": "attn_prefill_varlen", "achieved": round(pre_tflops, 2),
                             "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                             "frac": round(pre_tflops / BF16_PEAK_TFLOPS, 4),
                             "traffic": recorded_traffic("attn_prefill_qwen3_8b_prefix_hbm_traffic.md",
                                                         "attn_prefill.hip")},
        "kernels": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                    for k, v in kernels.items()},
        "cpu_baseline": cpu,
        "parity": ({"attn_decode_paged": cpu["parity"], "attn_prefill_varlen": cpu_pre["parity"],
                    "reference": "fp64 CPU oracle on the inputs and outputs of the timed steps"}
                   if cpu is not None and cpu_pre is not None else None),
        "sublayer_ops": ops,
        "qk_norm_rope_small": norm_small,
        "qwen3_0_6b": small,
        "decode_graph": ladder,
        "decode_graph_short": ladder_short,
        "decode_graph_stack": stack,
        "cpu_baseline_prefill": cpu_pre,
        "cpu_baseline_stages": cpu_st,
        "cpu_baseline_one_thread": cpu_one,
    }
    print(json.dumps(out), flush=True)


def copy_reference(torch, dev, log):
    """What a plain streaming kernel reaches on this device, for context beside the
    8 TB/s peak: a device-to-device copy of 1 GiB, bytes read + written per second,
    best of five.  (The decode only reads; a copy mixes reads and writes, which
    streams more slowly, so the decode's rate can exceed it.)"""
    src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream()

    def best(fn):
        fn()
        times = []
        for _ in range(5):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            ev[0].record(stream)
            fn()
            ev[1].record(stream)
            torch.cuda.synchronize()
            times.append(ev[0].elapsed_time(ev[1]))
        return min(times)

    copy_ms = best(lambda: dst.copy_(src))
    out = {"copy_GB/s": round(2 * src.numel() * 4 / (copy_ms * 1e-3) / 1e9, 1)}
    log(f"streaming reference: {out}")
    del src, dst
    return out


def qwen3_0_6b_shapes(pkv, torch, dev, to_dev, args, log):
    """Secondary numbers at the Qwen3-0.6B head counts (16 q / 8 kv): the varlen causal
    prefill on fresh K/V (8 sequences, lengths U[128, 2048]; small enough that launch and
    tail dominate) and the paged decode of 64 sequences (contexts U[512, 8192]).  Each
    attention call is timed alone with events over args.steps launches."""
    import workloads as wl
    D = 128
    out = {}
    stream = torch.cuda.current_stream()

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        gpu_lead(torch, 0.5 * args.steps)
        ev[0].record(stream)
        for _ in range(args.steps):
            fn()
        ev[1].record(stream)
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / args.steps

    w2 = wl.varlen_prefill(args.seed)
    s6 = w2.shape
    q0, k0, v0 = wl.qkv_views(s6)
    qkv = to_dev(w2.qkv())
    T = qkv.shape[0]
    q = qkv[:, q0:k0].view(T, s6.num_q_heads, D)
    k = qkv[:, k0:v0].view(T, s6.num_kv_heads, D)
    v = qkv[:, v0:].view(T, s6.num_kv_heads, D)
    cu = to_dev(w2.cu_seqlens)
    L = int(w2.lengths.max())
    o = torch.empty((T, s6.num_q_heads, D), dtype=torch.bfloat16, device=dev)
    ms = timed(lambda: pkv.attn_prefill_varlen(q, k, v, cu, cu, L, L, out=o))
    out["varlen_prefill"] = {"tokens": T, "lengths": [int(x) for x in w2.lengths], "ms": round(ms, 4),
                             "TFLOP/s": round(w2.flops / (ms * 1e-3) / 1e12, 2)}
    del qkv, o

    w3 = wl.paged_decode_0_6b(args.seed)
    hkv, hq = w3.shape.num_kv_heads, w3.shape.num_q_heads
    kc = torch.empty((w3.num_blocks, 256, hkv, D), dtype=torch.bfloat16, device=dev)
    vc = torch.empty_like(kc)
    wl.fill_normal_bf16_(kc, 3, args.seed, 10)
    wl.fill_normal_bf16_(vc, 3, args.seed, 11)
    qd, cl, bt = to_dev(w3.q()), to_dev(w3.context_lens), to_dev(w3.block_tables)
    ws = torch.empty(pkv.decode_workspace_bytes(w3.batch, hq, hkv, w3.block_tables.shape[1]), dtype=torch.uint8,
                     device=dev)
    od = torch.empty((w3.batch, hq, D), dtype=torch.bfloat16, device=dev)
    ms = timed(lambda: pkv.attn_decode_paged(qd, kc, vc, cl, bt, out=od, workspace=ws))
    nbytes = w3.algorithmic_bytes()
    out["paged_decode"] = {"batch": w3.batch, "ms": round(ms, 4), "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 2),
                           "bytes": nbytes}
    log(f"qwen3-0.6b shapes: {json.dumps(out)}")
    del kc, vc
    return out


def norm_rope_small(pkv, torch, dev, table, args, log):
    """QK-Norm + RoPE (the unfused pass) at the Qwen3-0.6B head counts (16 q / 8 kv) on
    the token counts of the small correctness workload (337) and of the 0.6B varlen
    prefill (its eight lengths): secondary HBM-bound numbers."""
    import workloads as wl
    s6 = wl.QWEN3_0_6B
    D = 128
    out = {}
    for label, T in (("tiny_337", 337), ("varlen_prefill", int(wl.varlen_prefill(args.seed).lengths.sum()))):
        gen = torch.Generator(device=dev)
        gen.manual_seed(args.seed + T)
        qkv = torch.randn((T, s6.qkv_width), generator=gen, device=dev).to(torch.bfloat16)
        q0, k0, v0 = wl.qkv_views(s6)
        q = qkv[:, q0:k0].view(T, s6.num_q_heads, D)
        k = qkv[:, k0:v0].view(T, s6.num_kv_heads, D)
        pos = torch.arange(T, dtype=torch.int64, device=dev) % 4096
        g = torch.ones(D, dtype=torch.bfloat16, device=dev)
        qo = torch.empty((T, s6.num_q_heads, D), dtype=torch.bfloat16, device=dev)
        ko = torch.empty((T, s6.num_kv_heads, D), dtype=torch.bfloat16, device=dev)
        fn = lambda: pkv.qk_norm_rope(q, k, pos, g, g, table, s6.eps, q_out=qo, k_out=ko)
        for _ in range(args.warmup):
            fn()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        gpu_lead(torch, 0.5 * args.steps)
        ev[0].record(torch.cuda.current_stream())
        for _ in range(args.steps):
            fn()
        ev[1].record(torch.cuda.current_stream())
        torch.cuda.synchronize()
        ms = ev[0].elapsed_time(ev[1]) / args.steps
        nbytes = T * ((s6.num_q_heads + s6.num_kv_heads) * D * 2 * 2 + 8 + 512)
        out[label] = {"tokens": T, "ms": round(ms, 4), "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 2), "bytes": nbytes}
    log(f"qk_norm_rope at 0.6B shapes: {json.dumps(out)}")
    return out


def sublayer_ops(pkv, torch, dev, to_dev, args, log):
    """The elementwise steps around attention at Qwen3-8B sizes, each timed alone with
    events over args.steps launches: residual add + RMSNorm on the prefill's 32768
    tokens (hidden 4096), SiluAndMul on 32768 tokens (intermediate 12288), and the
    sampler on the decode batch's 256 rows of 151936 bf16 logits (Philox noise)."""
    import workloads as wl
    T, H, I, B, V = 32768, wl.HIDDEN_8B, wl.INTERMEDIATE_8B, 256, wl.VOCAB
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed + 31)
    x = torch.randn((T, H), generator=gen, device=dev).to(torch.bfloat16)
    r = (3 * torch.randn((T, H), generator=gen, device=dev)).to(torch.bfloat16)
    g = (1 + 0.05 * torch.randn((H,), generator=gen, device=dev)).to(torch.bfloat16)
    y, r_out = torch.empty_like(x), torch.empty_like(x)
    gu = (2 * torch.randn((T, 2 * I), generator=gen, device=dev)).to(torch.bfloat16)
    act = torch.empty((T, I), dtype=torch.bfloat16, device=dev)
    lg_np, temps_np = wl.sampler_inputs(args.seed, B)
    lg, temps = to_dev(lg_np), to_dev(temps_np)
    tok = torch.empty(B, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream()
    cases = {
        "add_rms_norm": (lambda: pkv.add_rms_norm(x, r, g, 1e-6, y=y, residual_out=r_out), T * H * 2 * 4 + H * 2,
                         f"[{T}, {H}] bf16: read x, residual; write y, residual (32 KiB per token)"),
        "silu_and_mul": (lambda: pkv.silu_and_mul(gu, out=act), T * I * 2 * 3,
                         f"[{T}, 2 x {I}] bf16 -> [{T}, {I}]"),
        "sample_gumbel": (lambda: pkv.sample_gumbel(lg, temps, seed=1, offset=0, out=tok), B * V * 2 + B * 12,
                          f"[{B}, {V}] bf16 logits, in-kernel Philox4x32-10 noise"),
    }
    out = {}
    for name, (fn, nbytes, what) in cases.items():
        for _ in range(args.warmup):
            fn()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        gpu_lead(torch, 0.5 * args.steps)
        ev[0].record(stream)
        for _ in range(args.steps):
            fn()
        ev[1].record(stream)
        torch.cuda.synchronize()
        ms = ev[0].elapsed_time(ev[1]) / args.steps
        out[name] = {"ms": round(ms, 4), "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 2), "bytes": nbytes,
                     "shape": what}
    log(f"sublayer ops: {json.dumps(out)}")
    del x, r, y, r_out, gu, act
    return out


def decode_graph_ladder(pkv, torch, s8, table, qkv_d, kc_d, vc_d, pos_d, slot_d, cl_d, bt_d, gq_d, gk_d, args, log):
    """Decode step (QK-Norm + RoPE + scatter, paged decode) per batch bucket: eager vs HIP-graph replay.

    Batch B runs the first B sequences of the decode workload.  "latency": host wall
    time of one step from launch to completion (launch, then synchronise), averaged;
    "back_to_back": wall time of consecutive steps without synchronisation, per step.
    """
    B = qkv_d.shape[0]
    st = pkv.DecodeStep(qkv_d, kc_d, vc_d, pos_d, slot_d, cl_d, bt_d, gq_d, gk_d, table, s8.num_q_heads,
                        s8.num_kv_heads, eps=s8.eps)
    st.capture()
    reps = max(args.steps, 20)
    out = {"workload": "first B sequences of the decode workload, one step = qk_norm_rope_store + paged decode",
           "unit": "us/step", "latency": {"eager": {}, "graph": {}}, "back_to_back": {"eager": {}, "graph": {}}}
    for b in st.buckets:
        for mode, fn in (("eager", st.run), ("graph", st.replay)):
            for _ in range(3):
                fn(b)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(reps):
                fn(b)
                torch.cuda.synchronize()
            out["latency"][mode][str(b)] = round((time.perf_counter() - t0) * 1e6 / reps, 2)
            t0 = time.perf_counter()
            for _ in range(reps):
                fn(b)
            torch.cuda.synchronize()
            out["back_to_back"][mode][str(b)] = round((time.perf_counter() - t0) * 1e6 / reps, 2)
    st.close()
    log(f"decode graph ladder (us/step): {json.dumps(out)}")
    return out


def decode_graph_short(pkv, torch, dev, to_dev, table, args, log):
    """Decode step on short contexts (64 sequences, contexts U[256, 1024], 32/8 heads), where
    launch overhead rather than K/V bytes sets the time: eager vs HIP-graph replay per bucket
    B = 1 ... 64 (latency: launch then synchronise; back_to_back: consecutive steps), and at
    batches between buckets (3, 12, 48) the replay with the library's padding launch vs the
    caller keeping the padded rows itself (PKV_DECODE_CALLER_PADS)."""
    import workloads as wl
    w = wl.short_decode_8b(args.seed)
    s8 = w.shape
    kc = torch.empty((w.num_blocks, 256, s8.num_kv_heads, 128), dtype=torch.bfloat16, device=dev)
    vc = torch.empty_like(kc)
    wl.fill_normal_bf16_(kc, 6, args.seed, 10)
    wl.fill_normal_bf16_(vc, 6, args.seed, 11)
    qkv = to_dev(w.qkv())
    gq, gk = (to_dev(g) for g in w.gammas())
    pos, slot = to_dev(w.positions), to_dev(w.slot_mapping)
    cl, bt = to_dev(w.context_lens), to_dev(w.block_tables)
    reps = max(args.steps, 50)

    def timing(fn, b):
        for _ in range(5):
            fn(b)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            fn(b)
            torch.cuda.synchronize()
        lat = (time.perf_counter() - t0) * 1e6 / reps
        t0 = time.perf_counter()
        for _ in range(reps):
            fn(b)
        torch.cuda.synchronize()
        return round(lat, 2), round((time.perf_counter() - t0) * 1e6 / reps, 2)

    out = {"workload": f"{w.batch} sequences of the 8B shapes, contexts U[256, 1024] (mean "
                       f"{float(w.context_lens.mean()):.0f}); one step = qk_norm_rope_store + paged decode",
           "unit": "us/step", "latency": {"eager": {}, "graph": {}}, "back_to_back": {"eager": {}, "graph": {}},
           "between_buckets": {}}
    st = pkv.DecodeStep(qkv, kc, vc, pos, slot, cl, bt, gq, gk, table, s8.num_q_heads, s8.num_kv_heads, eps=s8.eps)
    st.capture()
    for b in st.buckets:
        for mode, fn in (("eager", st.run), ("graph", st.replay)):
            lat, btb = timing(fn, b)
            out["latency"][mode][str(b)] = lat
            out["back_to_back"][mode][str(b)] = btb
    st.close()
    # between buckets: the library pads rows [b, bucket) with one kernel per replay, or the
    # caller keeps them padded (slot -1, context 0) and the replay is the graph alone
    slot_p, cl_p = slot.clone(), cl.clone()
    stc = pkv.DecodeStep(qkv, kc, vc, pos, slot_p, cl_p, bt, gq, gk, table, s8.num_q_heads, s8.num_kv_heads,
                         eps=s8.eps, caller_pads=True)
    stc.capture()
    stl = pkv.DecodeStep(qkv, kc, vc, pos, slot.clone(), cl.clone(), bt, gq, gk, table, s8.num_q_heads,
                         s8.num_kv_heads, eps=s8.eps)
    stl.capture()
    for b in (3, 12, 48):
        n = stc.bucket(b)
        slot_p.copy_(slot)
        cl_p.copy_(cl)
        slot_p[b:n] = -1
        cl_p[b:n] = 0
        torch.cuda.synchronize()
        lat_l, btb_l = timing(stl.replay, b)
        lat_c, btb_c = timing(stc.replay, b)
        out["between_buckets"][str(b)] = {"bucket": n, "library_pads": {"latency": lat_l, "back_to_back": btb_l},
                                          "caller_pads": {"latency": lat_c, "back_to_back": btb_c}}
    stc.close()
    stl.close()
    log(f"decode graph, short contexts (us/step): {json.dumps(out)}")
    del kc, vc
    return out


def decode_graph_stack(pkv, torch, dev, to_dev, table, args, log, layers=36, batches=(1, 4, 16, 64)):
    """A layer stack of decode steps (Qwen3-8B has 36 layers, each with its own KV cache) on short
    contexts (contexts U[256, 1024], 32/8 heads), eager (2 launches per layer) against one HIP graph
    holding all layers' steps, captured through torch: latency (launch, then synchronise) and
    back_to_back, both per layer."""
    import workloads as wl
    w = wl.short_decode_8b(args.seed)
    s8 = w.shape
    kc0 = torch.empty((w.num_blocks, 256, s8.num_kv_heads, 128), dtype=torch.bfloat16, device=dev)
    vc0 = torch.empty_like(kc0)
    wl.fill_normal_bf16_(kc0, 6, args.seed, 10)
    wl.fill_normal_bf16_(vc0, 6, args.seed, 11)
    qkv = to_dev(w.qkv())
    gq, gk = (to_dev(g) for g in w.gammas())
    pos, slot = to_dev(w.positions), to_dev(w.slot_mapping)
    cl, bt = to_dev(w.context_lens), to_dev(w.block_tables)
    caches = [(kc0.clone(), vc0.clone()) for _ in range(layers)]
    steps = [pkv.DecodeStep(qkv, kc, vc, pos, slot, cl, bt, gq, gk, table, s8.num_q_heads, s8.num_kv_heads,
                            eps=s8.eps) for kc, vc in caches]
    reps = max(args.steps, 20)
    out = {"workload": f"{layers} layers, each its own KV cache; {w.batch} sequences of the 8B shapes, contexts "
                       f"U[256, 1024]; per layer: qk_norm_rope_store + paged decode", "layers": layers,
           "unit": "us/layer", "latency": {"eager": {}, "graph": {}}, "back_to_back": {"eager": {}, "graph": {}}}
    for b in batches:
        def eager(b=b):
            for st in steps:
                st.run(b)
        g = torch.cuda.CUDAGraph()
        eager()
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            eager()
        torch.cuda.synchronize()
        for mode, fn in (("eager", eager), ("graph", g.replay)):
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(reps):
                fn()
                torch.cuda.synchronize()
            out["latency"][mode][str(b)] = round((time.perf_counter() - t0) * 1e6 / reps / layers, 2)
            t0 = time.perf_counter()
            for _ in range(reps):
                fn()
            torch.cuda.synchronize()
            out["back_to_back"][mode][str(b)] = round((time.perf_counter() - t0) * 1e6 / reps / layers, 2)
        del g
    for st in steps:
        st.close()
    log(f"decode layer stack, eager vs one graph (us/layer): {json.dumps(out)}")
    del caches, kc0, vc0
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_stages(args, wp, qkv_p, log):
    """The oracle's first two steps on the first 16384 tokens of the prefix-hit prefill:
    QK-Norm + RoPE of q and k, then the scatter of k' and v into a host cache.  GB/s of the
    same algorithmic bytes the GPU kernels are credited with."""
    import torch

    import oracle
    import workloads as wl
    s8 = wl.QWEN3_8B
    n = min(16384, wp.num_q_tokens)
    qkv = qkv_p[:n].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    q0, k0, v0 = wl.qkv_views(s8)
    gq, gk = wp.gammas()
    pos = np.ascontiguousarray(wp.positions[:n])
    table = oracle.rope_table(s8.max_position, 128, s8.rope_theta)
    t0 = time.perf_counter()
    oracle.rmsnorm_rope(qkv, s8.num_q_heads, 128, gq, s8.eps, pos, table, col_offset=q0)
    kr = oracle.rmsnorm_rope(qkv, s8.num_kv_heads, 128, gk, s8.eps, pos, table, col_offset=k0)
    t_norm = time.perf_counter() - t0
    kb = oracle.round_bf16(kr)
    vb = np.ascontiguousarray(qkv[:, v0:]).reshape(n, s8.num_kv_heads, 128)
    kc = np.zeros((wp.num_blocks * 256, s8.num_kv_heads, 128), np.uint16)
    vc = np.zeros_like(kc)
    t0 = time.perf_counter()
    oracle.store_kvcache(kb, vb, kc, vc, np.ascontiguousarray(wp.slot_mapping[:n]))
    t_store = time.perf_counter() - t0
    norm_bytes = n * ((s8.num_q_heads + s8.num_kv_heads) * 128 * 2 * 2 + 8 + 512)
    store_bytes = n * (2 * 2 * 2 * s8.num_kv_heads * 128 + 4)
    out = {"qk_norm_rope": {"value": round(norm_bytes / t_norm / 1e9, 4), "unit": "GB/s", "s": round(t_norm, 3)},
           "store_kvcache": {"value": round(store_bytes / t_store / 1e9, 4), "unit": "GB/s", "s": round(t_store, 3)},
           "cores": oracle.num_threads(), "kind": "oracle",
           "sample": f"first {n} tokens of the prefix-hit prefill, 32/8 heads, fp64 C oracle"}
    log(f"cpu stages: {json.dumps(out)}")
    return out


def cpu_one_thread(args, log):
    """The oracle on one host thread for the small configurations: the whole tiny chain
    (QK-Norm + RoPE of q and k, the scatter, case-1 prefill; 337 tokens at 16/8 heads), 2048
    random (token, head) rows of the 0.6B varlen prefill and 8 sequences of the 0.6B decode
    batch.  Inputs are generated on the host (untimed); only the oracle calls are timed."""
    import oracle
    import workloads as wl
    prev = oracle.num_threads()
    oracle.set_num_threads(1)
    try:
        out = {}
        w = wl.tiny_chain(args.seed)
        s = w.shape
        q0, k0, v0 = wl.qkv_views(s)
        hq, hkv = s.num_q_heads, s.num_kv_heads
        table = oracle.rope_table(s.max_position, 128, s.rope_theta)
        t0 = time.perf_counter()
        qb = oracle.round_bf16(oracle.rmsnorm_rope(w.qkv, hq, 128, w.gamma_q, s.eps, w.positions, table,
                                                   col_offset=q0))
        kb = oracle.round_bf16(oracle.rmsnorm_rope(w.qkv, hkv, 128, w.gamma_k, s.eps, w.positions, table,
                                                   col_offset=k0))
        vb = np.ascontiguousarray(w.qkv[:, v0:]).reshape(-1, hkv, 128)
        kc = np.zeros((w.num_blocks * 256, hkv, 128), np.uint16)
        vc = np.zeros_like(kc)
        oracle.store_kvcache(kb, vb, kc, vc, w.slot_mapping)
        oracle.attn_prefill(qb, kb, vb, w.cu_seqlens, w.cu_seqlens, hq, hkv)
        dt = time.perf_counter() - t0
        T = int(sum(w.lengths))
        out["tiny_chain"] = {"value": round(T / dt, 1), "unit": "tokens/s", "s": round(dt, 4),
                             "sample": f"whole chain, {T} tokens, {hq}/{hkv} heads"}

        w2 = wl.varlen_prefill(args.seed)
        s2 = w2.shape
        q0, k0, v0 = wl.qkv_views(s2)
        qkv = w2.qkv()
        n2 = qkv.shape[0]
        q = np.ascontiguousarray(qkv[:, q0:k0]).reshape(n2, s2.num_q_heads, 128)
        k = np.ascontiguousarray(qkv[:, k0:v0]).reshape(n2, s2.num_kv_heads, 128)
        v = np.ascontiguousarray(qkv[:, v0:]).reshape(n2, s2.num_kv_heads, 128)
        rng = np.random.default_rng(args.seed + 300)
        t = rng.integers(0, n2, 2048)
        rows = np.stack([t, rng.integers(0, s2.num_q_heads, 2048)], 1)
        t0 = time.perf_counter()
        oracle.attn_prefill(q, k, v, w2.cu_seqlens, w2.cu_seqlens, s2.num_q_heads, s2.num_kv_heads, rows=rows)
        dt = time.perf_counter() - t0
        flop = float(np.sum(4 * 128 * (w2.positions[t] + 1)))
        out["varlen_prefill_0_6b"] = {"value": round(flop / dt / 1e9, 4), "unit": "GFLOP/s", "s": round(dt, 4),
                                      "sample": "2048 random (token, head) rows of the 8-sequence batch"}

        w3 = wl.paged_decode_0_6b(args.seed)
        s3 = w3.shape
        seqs = list(range(8))
        cl = w3.context_lens[seqs].astype(np.int32)
        nblk = [-(-int(c) // 256) for c in cl]
        rows_bt, nxt = [], 0
        for nb in nblk:
            rows_bt.append(list(range(nxt, nxt + nb)))
            nxt += nb
        bt = wl.pad_block_tables(rows_bt, w3.block_tables.shape[1])
        rng = wl.rng_for(3, args.seed, 40)
        kc = wl.normal_bf16(rng, (nxt * 256, s3.num_kv_heads, 128))
        vc = wl.normal_bf16(rng, (nxt * 256, s3.num_kv_heads, 128))
        qd = w3.q()[seqs]
        t0 = time.perf_counter()
        oracle.attn_decode(qd, kc, vc, cl, bt, s3.num_q_heads, s3.num_kv_heads)
        dt = time.perf_counter() - t0
        nbytes = int(np.sum(cl.astype(np.int64))) * s3.num_kv_heads * 128 * 4 + len(seqs) * s3.num_q_heads * 512
        out["paged_decode_0_6b"] = {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "s": round(dt, 4),
                                    "sample": f"{len(seqs)} of the {w3.batch} sequences "
                                              f"({int(cl.sum())} context tokens)"}
        out.update({"cores": oracle.num_threads(), "kind": "oracle"})
    finally:
        oracle.set_num_threads(prev)
    log(f"cpu one-thread: {json.dumps(out)}")
    return out


def cpu_baseline(args, wd, kc_d, vc_d, q_d, o_d, log):
    """The oracle's paged decode over the decode workload's sequences, on the host cores.

    Sequences are copied back and run in groups of 32 so host memory stays bounded;
    only the oracle calls are timed.  Units: GB/s of the same algorithmic bytes.
    """
    import torch

    import oracle
    import workloads as wl

    def bits(t):
        return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    def gather_sequences(seqs):
        rows = [[int(x) for x in wd.block_tables[b, :-(-int(wd.context_lens[b]) // 256)]] for b in seqs]
        uniq = sorted({p for r in rows for p in r})
        where = {p: i for i, p in enumerate(uniq)}
        idx = torch.tensor(uniq, dtype=torch.int64, device=kc_d.device)
        hkv = kc_d.shape[2]
        kc = bits(kc_d.index_select(0, idx)).reshape(len(uniq) * 256, hkv, 128)
        vc = bits(vc_d.index_select(0, idx)).reshape(len(uniq) * 256, hkv, 128)
        return kc, vc, wl.pad_block_tables([[where[p] for p in r] for r in rows], wd.block_tables.shape[1])

    n = min(args.cpu_seqs, wd.batch)
    seqs_all = list(range(n))
    qh = bits(q_d)
    got = bits(o_d).astype(np.uint32) << 16
    got = got.view(np.float32).astype(np.float64)
    hq, hkv = wd.shape.num_q_heads, wd.shape.num_kv_heads
    total, logical, toks = 0.0, 0, 0
    err_max, err_sum, err_n = 0.0, 0.0, 0
    for s0 in range(0, n, 32):
        seqs = seqs_all[s0:s0 + 32]
        kc, vc, bt = gather_sequences(seqs)
        cl = wd.context_lens[seqs]
        t0 = time.perf_counter()
        ref = oracle.attn_decode(qh[seqs], kc, vc, cl, bt, hq, hkv)
        total += time.perf_counter() - t0
        err = np.abs(got[seqs] - ref)
        err_max, err_sum, err_n = max(err_max, float(err.max())), err_sum + float(err.sum()), err_n + err.size
        toks += int(np.sum(cl.astype(np.int64)))
        logical += int(np.sum(cl.astype(np.int64))) * hkv * 128 * 2 * 2 + len(seqs) * hq * 128 * 2 * 2
        del kc, vc
    # the same algorithmic bytes as the GPU figure (shared prefix once) when the whole batch ran
    unique = wd.algorithmic_bytes(unique=True) if n == wd.batch else None
    nbytes = unique if unique is not None else logical
    log(f"cpu baseline: {n} sequences, {nbytes / 1e9:.3f} GB in {total:.2f} s; GPU vs oracle max |err| "
        f"{err_max:.3e} mean {err_sum / err_n:.3e}")
    parity = {"max_abs": err_max, "mean_abs": err_sum / err_n, "compared": f"all {hq} heads of {n} sequences",
              "gate": {"max_abs": 2e-2, "mean_abs": 2e-3},
              "pass": bool(err_max <= 2e-2 and err_sum / err_n <= 2e-3)}
    return {"value": round(nbytes / total / 1e9, 4), "unit": "GB/s", "cores": oracle.num_threads(), "kind": "oracle",
            "cpu_model": cpu_model(), "logical_GB/s": round(logical / total / 1e9, 4),
            "sample": f"paged decode of {n} of the {wd.batch} sequences ({toks} context tokens, {hq}/{hkv} heads), "
                      f"fp64 C oracle with OpenMP, {total:.2f} s of oracle time; value in the GPU figure's bytes "
                      f"({'shared prefix counted once' if unique is not None else 'K/V per sequence'}), "
                      f"logical_GB/s with the prefix counted per sequence as the oracle reads it",
            "parity": parity}


def cpu_baseline_prefill(args, wp, kc_p, vc_p, q_p, o_p, log):
    """The oracle's paged prefill on a sample of (token, head) rows of the prefill workload,
    compared with the same rows of the output the GPU produced in the timed steps."""
    import torch

    import oracle

    def bits(t):
        return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    rng = np.random.default_rng(args.seed + 200)
    nrows = args.cpu_prefill_rows
    t = rng.integers(0, wp.num_q_tokens, nrows)
    h = rng.integers(0, wp.shape.num_q_heads, nrows)
    rows = np.stack([t, h], 1)
    kc, vc = bits(kc_p).reshape(-1, 8, 128), bits(vc_p).reshape(-1, 8, 128)
    qh = bits(q_p)
    t0 = time.perf_counter()
    ref = oracle.attn_prefill(qh, kc, vc, wp.cu_seqlens_q, wp.cu_seqlens_k, wp.shape.num_q_heads,
                              wp.shape.num_kv_heads, block_table=wp.block_tables, rows=rows)
    dt = time.perf_counter() - t0
    got = (bits(o_p)[t, h].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    err = np.abs(got - ref)
    flop = float(np.sum(4 * 128 * (wp.positions[t] + 1)))
    log(f"cpu prefill baseline: {nrows} rows, {flop / 1e9:.2f} GFLOP in {dt:.2f} s; GPU vs oracle max |err| "
        f"{err.max():.3e} mean {err.mean():.3e}")
    parity = {"max_abs": float(err.max()), "mean_abs": float(err.mean()),
              "compared": f"{nrows} random (token, head) rows of {wp.num_q_tokens * wp.shape.num_q_heads}",
              "gate": {"max_abs": 2e-2, "mean_abs": 2e-3},
              "pass": bool(err.max() <= 2e-2 and err.mean() <= 2e-3)}
    return {"value": round(flop / dt / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{nrows} random (token, head) rows of the prefix-hit prefill, fp64 C oracle, {dt:.2f} s",
            "parity": parity}


if __name__ == "__main__":
    main()
