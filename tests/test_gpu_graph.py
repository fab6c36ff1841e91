"""GPU parity of the decode step and its HIP-graph replay per batch bucket.

A run of decode steps with changing batch sizes (most of them between two
buckets, so the graph pads rows with slot -1 / context 0) is played three ways
on the same seeded inputs:
  * graph replay  (DecodeStep.replay(b): pad rows [b, bucket), launch the graph)
  * eager         (DecodeStep.run(bucket) on inputs the test pads the same way)
  * the oracle    (QK-Norm + RoPE, scatter and paged decode in fp64 on a host
                   copy of the pool, rows < b only)
Graph and eager must agree byte for byte (outputs and both caches); both must
meet the attention gate against the oracle.  Eager torch work and host
synchronisations sit between the replays, and every replay is checked.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_gqa_amd as pkv
import workloads as wl
from gpu_helpers import bits, check_attn, f64, to_dev

pytestmark = pytest.mark.gpu
D = 128


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pkv.load_library()
    return torch.device("cuda:0")


def _say(*a):
    print("[gpu]", *a, flush=True)


class _Sequences:
    """max_batch sequences, each with its own blocks, growing by one token per step."""

    def __init__(self, max_batch, max_ctx, steps, seed):
        rng = wl.rng_for(93, seed, 0)
        self.ctx0 = rng.integers(1, max_ctx - steps, size=max_batch).astype(np.int64)
        self.mb = -(-max_ctx // 256)
        self.num_blocks = max_batch * self.mb + 3
        perm = rng.permutation(self.num_blocks)[:max_batch * self.mb]
        self.block_tables = perm.reshape(max_batch, self.mb).astype(np.int32)
        self.rng = rng

    def step_inputs(self, k, shape, max_batch, b):
        """Inputs of step k for the first b rows; rows >= b hold junk the step must ignore."""
        ctx = self.ctx0 + k + 1                       # tokens in cache once this step's token is stored
        pos = ctx - 1
        slots = np.array([self.block_tables[i, pos[i] // 256] * 256 + pos[i] % 256 for i in range(max_batch)],
                         np.int32)
        qkv = wl.normal_bf16(self.rng, (max_batch, shape.qkv_width))
        # junk in the padded rows: the graph launch must overwrite slot / context itself
        slots[b:] = 0
        ctx_i32 = ctx.astype(np.int32)
        ctx_i32[b:] = 7
        return qkv, pos.astype(np.int64), slots, ctx_i32


@pytest.mark.parametrize("hq,hkv,max_batch,max_ctx,batches,caller_pads", [
    (32, 8, 32, 1000, [3, 32, 17, 1, 9, 5], False),
    (16, 8, 32, 1000, [3, 32, 17, 1, 9, 5], False),
    (32, 8, 512, 256, [512, 300, 257, 1, 129], False),   # the whole ladder 1 ... 512, batches past a bucket edge
    (32, 8, 32, 1000, [3, 32, 17, 1, 9, 5], True),       # the caller pads rows [b, bucket); no padding launch
])
def test_decode_graph_replays_match_eager_and_oracle(dev, hq, hkv, max_batch, max_ctx, batches, caller_pads):
    shape = wl.QWEN3_8B if hq == 32 else wl.QWEN3_0_6B
    _say(f"decode graph {hq}/{hkv} heads, max_batch {max_batch}, batches {batches}, caller pads: {caller_pads}")
    seqs = _Sequences(max_batch, max_ctx, len(batches), seed=hq + max_batch)
    rng = wl.rng_for(94, hq, 0)
    pool0 = wl.normal_bf16(rng, (2, seqs.num_blocks, 256, hkv, D))
    gq, gk = wl.gamma_bf16(rng), wl.gamma_bf16(rng)
    table_h = oracle.rope_table(40960, D, 1e6)
    table_d = pkv.rope_cache_build(40960, D, 1e6, device=dev)
    gq_d, gk_d = to_dev(gq, dev), to_dev(gk, dev)

    def make():
        bufs = dict(qkv=torch.zeros((max_batch, shape.qkv_width), dtype=torch.bfloat16, device=dev),
                    kc=to_dev(pool0[0], dev), vc=to_dev(pool0[1], dev),
                    pos=torch.zeros(max_batch, dtype=torch.int64, device=dev),
                    slot=torch.zeros(max_batch, dtype=torch.int32, device=dev),
                    ctx=torch.zeros(max_batch, dtype=torch.int32, device=dev),
                    bt=to_dev(seqs.block_tables, dev))
        st = pkv.DecodeStep(bufs["qkv"], bufs["kc"], bufs["vc"], bufs["pos"], bufs["slot"], bufs["ctx"], bufs["bt"],
                            gq_d, gk_d, table_d, hq, hkv, eps=shape.eps, caller_pads=caller_pads)
        return st, bufs

    graph, gb = make()
    eager, eb = make()
    graph.capture()
    assert graph.buckets == tuple(1 << i for i in range(max_batch.bit_length()))
    ek, ev = pool0[0].reshape(-1, hkv, D).copy(), pool0[1].reshape(-1, hkv, D).copy()
    q0, k0, v0 = wl.qkv_views(shape)

    for k, b in enumerate(batches):
        n = graph.bucket(b)
        assert n == next(x for x in graph.buckets if x >= b)
        qkv, pos, slots, ctx = seqs.step_inputs(k, shape, max_batch, b)
        ps, pc = slots.copy(), ctx.copy()
        ps[b:n], pc[b:n] = -1, 0
        # graph: junk rows as given and the launch pads them, or the caller pads them
        for buf, x in ((gb["qkv"], qkv), (gb["pos"], pos), (gb["slot"], ps if caller_pads else slots),
                       (gb["ctx"], pc if caller_pads else ctx)):
            buf.copy_(to_dev(x, dev))
        graph.replay(b)
        # eager at the bucket size with the padding written by the test
        for buf, x in ((eb["qkv"], qkv), (eb["pos"], pos), (eb["slot"], ps), (eb["ctx"], pc)):
            buf.copy_(to_dev(x, dev))
        eager.run(n)
        # unrelated eager work between replays
        junk = torch.randn(1 << 20, device=dev).sum()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)

        tag = f"step {k} batch {b} bucket {n}"
        assert torch.equal(graph.o[:n].view(torch.int16), eager.o[:n].view(torch.int16)), f"{tag}: o"
        assert torch.equal(gb["kc"].view(torch.int16), eb["kc"].view(torch.int16)), f"{tag}: k_cache"
        assert torch.equal(gb["vc"].view(torch.int16), eb["vc"].view(torch.int16)), f"{tag}: v_cache"
        assert gb["slot"][b:n].eq(-1).all() and gb["ctx"][b:n].eq(0).all(), f"{tag}: padding"
        if n > b:
            assert graph.o[b:n].float().abs().max().item() == 0.0, f"{tag}: padded rows must be zero"

        # oracle on rows < b
        rq = oracle.round_bf16(oracle.rmsnorm_rope(qkv[:b], hq, D, gq, shape.eps, pos[:b], table_h, col_offset=q0))
        rk = oracle.round_bf16(oracle.rmsnorm_rope(qkv[:b], hkv, D, gk, shape.eps, pos[:b], table_h, col_offset=k0))
        rv = np.ascontiguousarray(qkv[:b, v0:]).reshape(b, hkv, D)
        oracle.store_kvcache(rk, rv, ek, ev, slots[:b])
        ref = oracle.attn_decode(rq, ek, ev, ctx[:b], seqs.block_tables[:b], hq, hkv)
        check_attn(f64(graph.o[:b]), ref, tag)
        # value rows are copies: bit-exact against the oracle's scatter
        assert np.array_equal(bits(gb["vc"]).reshape(ev.shape)[slots[:b]], ev[slots[:b]]), f"{tag}: v rows"
    graph.close()


def test_decode_graph_batch_above_largest_bucket_is_refused(dev):
    _say("decode graph: batch above the largest bucket")
    shape = wl.QWEN3_0_6B
    mb = 8
    qkv = torch.zeros((mb, shape.qkv_width), dtype=torch.bfloat16, device=dev)
    kc = torch.zeros((4, 256, 8, D), dtype=torch.bfloat16, device=dev)
    st = pkv.DecodeStep(qkv, kc, torch.zeros_like(kc), torch.zeros(mb, dtype=torch.int64, device=dev),
                        torch.full((mb,), -1, dtype=torch.int32, device=dev),
                        torch.zeros(mb, dtype=torch.int32, device=dev),
                        torch.zeros((mb, 4), dtype=torch.int32, device=dev),
                        torch.ones(D, dtype=torch.bfloat16, device=dev), torch.ones(D, dtype=torch.bfloat16, device=dev),
                        pkv.rope_cache_build(4096, D, 1e6, device=dev), 16, 8)
    st.capture([1, 2, 4])
    with pytest.raises(pkv.PkvError):
        st.replay(5)
    st.replay(0)
    st.replay(3)
    torch.cuda.synchronize()
    assert st.o[:4].float().abs().max().item() == 0.0        # every row has context 0
    st.close()


@pytest.mark.parametrize("hq,hkv,batch,max_ctx", [
    (32, 8, 5, 1000),     # short contexts, small batch: 64-key splits
    (16, 8, 9, 3000),     # G = 2
    (8, 8, 3, 700),       # G = 1
    (64, 8, 2, 600),      # G = 8
    (32, 8, 300, 2100),   # a grid past the chip: size-ordered dispatch
])
def test_decode_step_equals_the_two_calls(dev, hq, hkv, batch, max_ctx):
    """The step runs QK-Norm + RoPE + scatter inside the decode split kernel; its q',
    caches and output must equal, byte for byte, QK-Norm + RoPE + scatter followed by
    the decode call on the same inputs.  The batch holds a padded row (slot -1,
    context 0), a row with an empty context whose token is still stored, and contexts
    whose last key falls on every row of a 16-key chunk."""
    shape = wl.QWEN3_8B if hq == 32 else wl.QWEN3_0_6B
    width = (hq + 2 * hkv) * D
    _say(f"decode step vs two calls: {hq}/{hkv} heads, batch {batch}, contexts < {max_ctx}")
    rng = wl.rng_for(96, hq + batch, 0)
    mb = -(-max_ctx // 256)
    nb = batch * mb + 2
    perm = rng.permutation(nb)[:batch * mb]
    bt = perm.reshape(batch, mb).astype(np.int32)
    ctx = rng.integers(1, max_ctx, size=batch).astype(np.int64)
    ctx[:min(batch, 16)] = 17 * np.arange(min(batch, 16)) + 1   # key ctx - 1 on row i of its 16-key chunk
    ctx = np.minimum(ctx, max_ctx - 1)
    pos = ctx - 1
    slots = np.array([bt[i, pos[i] // 256] * 256 + pos[i] % 256 for i in range(batch)], np.int32)
    ctx32 = ctx.astype(np.int32)
    slots[batch - 1], ctx32[batch - 1] = -1, 0            # a padded row
    if batch > 2:
        ctx32[batch - 2] = 0                               # no context, the token is still stored
    qkv = wl.normal_bf16(rng, (batch, width))
    pool = wl.normal_bf16(rng, (2, nb, 256, hkv, D))
    gq, gk = wl.gamma_bf16(rng), wl.gamma_bf16(rng)
    table = pkv.rope_cache_build(40960, D, 1e6, device=dev)
    gq_d, gk_d = to_dev(gq, dev), to_dev(gk, dev)
    qkv_d, pos_d, slot_d, ctx_d, bt_d = (to_dev(x, dev) for x in (qkv, pos, slots, ctx32, bt))

    kc1, vc1 = to_dev(pool[0], dev), to_dev(pool[1], dev)
    st = pkv.DecodeStep(qkv_d, kc1, vc1, pos_d, slot_d, ctx_d, bt_d, gq_d, gk_d, table, hq, hkv, eps=shape.eps)
    st.run(batch)

    kc2, vc2 = to_dev(pool[0], dev), to_dev(pool[1], dev)
    q0, k0, v0 = hq * D, (hq + hkv) * D, width
    qv = qkv_d[:, :q0].view(batch, hq, D)
    kv = qkv_d[:, q0:k0].view(batch, hkv, D)
    vv = qkv_d[:, k0:v0].view(batch, hkv, D)
    q_out = pkv.qk_norm_rope_store(qv, kv, vv, pos_d, gq_d, gk_d, table, kc2, vc2, slot_d, eps=shape.eps)
    o2 = pkv.attn_decode_paged(q_out, kc2, vc2, ctx_d, bt_d)
    torch.cuda.synchronize()
    assert torch.equal(st.q_out[:batch].view(torch.int16), q_out.view(torch.int16)), "q'"
    assert torch.equal(kc1.view(torch.int16), kc2.view(torch.int16)), "k_cache"
    assert torch.equal(vc1.view(torch.int16), vc2.view(torch.int16)), "v_cache"
    assert torch.equal(st.o[:batch].view(torch.int16), o2.view(torch.int16)), "o"
    st.close()


def test_decode_steps_captured_by_the_caller_in_one_graph(dev):
    """A caller may capture several decode steps (here three layers, each with its own
    caches) into one graph of its own through torch: every replay (torch work and host
    synchronisations between them) gives, byte for byte, the eager steps' q', o and caches."""
    shape, hq, hkv, batch, layers = wl.QWEN3_0_6B, 16, 8, 5, 3
    _say(f"decode steps of {layers} layers captured into one caller graph, batch {batch}")
    rng = wl.rng_for(97, 0, 0)
    max_ctx, width = 900, (hq + 2 * hkv) * D
    mb = -(-max_ctx // 256)
    nb = batch * mb + 2
    bt = rng.permutation(nb)[:batch * mb].reshape(batch, mb).astype(np.int32)
    ctx = rng.integers(1, max_ctx, size=batch).astype(np.int64)
    pos = ctx - 1
    slots = np.array([bt[i, pos[i] // 256] * 256 + pos[i] % 256 for i in range(batch)], np.int32)
    table = pkv.rope_cache_build(40960, D, 1e6, device=dev)
    qkv_d = to_dev(wl.normal_bf16(rng, (batch, width)), dev)
    gq_d, gk_d = to_dev(wl.gamma_bf16(rng), dev), to_dev(wl.gamma_bf16(rng), dev)
    pos_d, slot_d, ctx_d, bt_d = (to_dev(x, dev) for x in (pos, slots, ctx.astype(np.int32), bt))
    pools = [wl.normal_bf16(rng, (2, nb, 256, hkv, D)) for _ in range(layers)]

    def make():
        caches = [(to_dev(p[0], dev), to_dev(p[1], dev)) for p in pools]
        steps = [pkv.DecodeStep(qkv_d, kc, vc, pos_d, slot_d, ctx_d, bt_d, gq_d, gk_d, table, hq, hkv, eps=shape.eps)
                 for kc, vc in caches]
        return caches, steps

    ref_caches, ref_steps = make()
    for st in ref_steps:
        st.run(batch)
    torch.cuda.synchronize()

    caches, steps = make()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for st in steps:
            st.run(batch)
    torch.cuda.synchronize()
    for rep in range(3):
        g.replay()
        torch.cuda.synchronize()
        for i in range(layers):
            assert torch.equal(steps[i].q_out[:batch].view(torch.int16), ref_steps[i].q_out[:batch].view(torch.int16)), \
                f"q' layer {i} replay {rep}"
            assert torch.equal(steps[i].o[:batch].view(torch.int16), ref_steps[i].o[:batch].view(torch.int16)), \
                f"o layer {i} replay {rep}"
            for c, rc in zip(caches[i], ref_caches[i]):
                assert torch.equal(c.view(torch.int16), rc.view(torch.int16)), f"cache layer {i} replay {rep}"
        for st in steps:                      # eager work between the replays overwrites the outputs
            st.o.zero_()
            st.q_out.zero_()
        torch.cuda.synchronize()
    for st in steps + ref_steps:
        st.close()
