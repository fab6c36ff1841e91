"""bench.py command-line contract that needs no GPU: a multi-GPU request is refused
with a message and a non-zero status before anything touches a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps", "1"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_recorded_traffic_follows_the_kernel_source(tmp_path, monkeypatch):
    """The committed traffic figures resolve for the current kernel sources, and a
    profile whose recorded source hash differs from the source gives null."""
    sys.path.insert(0, ROOT)
    import bench
    for prof, src in (("attn_decode_paged_qwen3_8b_hbm_traffic.md", "attn_decode.hip"),
                      ("attn_prefill_qwen3_8b_prefix_hbm_traffic.md", "attn_prefill.hip")):
        v = bench.recorded_traffic(prof, src)
        assert isinstance(v, int) and v > 0, f"{prof} does not match {src}: profile it again"
    (tmp_path / "profiles").mkdir()
    (tmp_path / "paged_kv_gqa_amd" / "csrc").mkdir(parents=True)
    (tmp_path / "paged_kv_gqa_amd" / "csrc" / "k.hip").write_text("kernel source\n")
    (tmp_path / "profiles" / "p.md").write_text("traffic_bytes_per_launch: 123\nsource_sha256: " + "0" * 64 + "\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.recorded_traffic("p.md", "k.hip") is None
    assert bench.recorded_traffic("missing.md", "k.hip") is None


def test_recorded_traffic_is_one_call_of_the_workload():
    """Each committed traffic figure is that of one call of the timed workload: the
    measured HBM bytes sit just above the bytes the call must move (decode: the
    unique K/V bytes; prefill: q, o and every cached K/V byte once), not a sum over
    several calls or workloads."""
    sys.path.insert(0, ROOT)
    import bench
    import workloads as wl
    dec = bench.recorded_traffic("attn_decode_paged_qwen3_8b_hbm_traffic.md", "attn_decode.hip")
    alg = wl.paged_decode_8b(0).algorithmic_bytes(True)
    assert 1.0 <= dec / alg <= 1.1, f"decode traffic {dec} is {dec / alg:.3f}x the call's bytes"
    wp = wl.prefix_prefill_8b(0)
    compulsory = wp.num_q_tokens * 32 * 128 * 2 * 2 + (wp.prefix_len + wp.num_seqs * wp.suffix_len) * 8 * 128 * 2 * 2
    pre = bench.recorded_traffic("attn_prefill_qwen3_8b_prefix_hbm_traffic.md", "attn_prefill.hip")
    assert 1.0 <= pre / compulsory <= 1.5, f"prefill traffic {pre} is {pre / compulsory:.3f}x the compulsory bytes"


def test_input_checksum_sees_every_word():
    """The checksum recorded beside the seed changes when any one input word changes,
    and not when nothing does."""
    import torch
    sys.path.insert(0, ROOT)
    import bench
    a = torch.arange(1 << 12, dtype=torch.int32).view(torch.bfloat16)
    b = torch.arange(100, dtype=torch.int64)
    ref = bench.input_checksum(torch, [("a", a), ("b", b)])
    assert ref == bench.input_checksum(torch, [("a", a.clone()), ("b", b.clone())])
    for i in (0, 1234, a.numel() - 1):
        a2 = a.clone()
        a2.view(torch.int16)[i] += 1
        assert bench.input_checksum(torch, [("a", a2), ("b", b)]) != ref
    assert bench.input_checksum(torch, [("a", a), ("b", b + 1)]) != ref
    assert bench.input_checksum(torch, [("b", b), ("a", a)]) != ref
    # a permutation keeps the plain sum but not the position-weighted one
    for i, j in ((0, 1), (5, 5 + (1 << 16)), (7, b.numel() - 1)):
        if j >= b.numel():
            continue
        b2 = b.clone()
        b2[i], b2[j] = b[j], b[i]
        assert bench.input_checksum(torch, [("a", a), ("b", b2)]) != ref
    a3 = a.clone().view(torch.int32)
    a3[[3, 1000]] = a3[[1000, 3]]
    assert bench.input_checksum(torch, [("a", a3.view(torch.bfloat16)), ("b", b)]) != ref
