"""Seeded input generators: determinism and metadata invariants (CPU only)."""
import numpy as np

import workloads as wl


def _check_tables(bt, lens, num_blocks, bs=256):
    for b, L in enumerate(lens):
        nb = -(-int(L) // bs)
        row = bt[b]
        assert np.all(row[:nb] >= 0) and np.all(row[:nb] < num_blocks)
        assert np.all(row[nb:] == -1)


def test_tiny_chain_layout_and_determinism():
    a, b = wl.tiny_chain(seed=0), wl.tiny_chain(seed=0)
    assert np.array_equal(a.qkv, b.qkv) and np.array_equal(a.block_tables, b.block_tables)
    assert a.qkv.shape == (337, 4096) and a.qkv.dtype == np.uint16
    assert list(a.cu_seqlens) == [0, 37, 337]
    _check_tables(a.block_tables, [41, 304], 8)
    assert a.block_tables.shape == (2, 2) and a.block_tables[0, 1] == -1
    # every written slot is distinct, in range, and inside the owning sequence's blocks
    slots = np.concatenate([a.slot_mapping] + [s.slot_mapping for s in a.decode_steps])
    assert len(np.unique(slots)) == len(slots) and slots.min() >= 0 and slots.max() < 8 * 256
    for j, st in enumerate(a.decode_steps):
        assert list(st.positions) == [37 + j, 300 + j]
        assert list(st.context_lens) == [38 + j, 301 + j]
    c = wl.tiny_chain(seed=1)
    assert not np.array_equal(a.qkv, c.qkv)


def test_varlen_prefill_workload():
    w = wl.varlen_prefill(seed=0)
    assert len(w.lengths) == 8 and w.lengths.min() >= 128 and w.lengths.max() <= 2048
    assert w.cu_seqlens[-1] == w.lengths.sum() == len(w.slot_mapping)
    _check_tables(w.block_tables, w.lengths, 4096)
    assert len(np.unique(w.slot_mapping)) == len(w.slot_mapping)
    expected = 4 * 128 * 16 * np.sum(w.lengths * (w.lengths + 1) / 2)
    assert w.flops == expected


def test_paged_decode_workloads():
    w3 = wl.paged_decode_0_6b(seed=0)
    assert w3.batch == 64 and w3.context_lens.min() >= 512 and w3.context_lens.max() <= 8192
    _check_tables(w3.block_tables, w3.context_lens, w3.num_blocks)
    assert w3.block_tables.shape == (64, 32)
    used = w3.block_tables[w3.block_tables >= 0]
    assert len(np.unique(used)) == len(used)            # no sharing in this workload
    w4 = wl.paged_decode_8b(seed=0)
    assert w4.batch == 256 and w4.block_tables.shape == (256, 128)
    assert w4.context_lens.min() >= 1024 and w4.context_lens.max() <= 32768
    _check_tables(w4.block_tables, w4.context_lens, w4.num_blocks)
    assert len(w4.shared_seqs) == 64 and len(w4.shared_blocks) == 8
    for b in w4.shared_seqs:
        assert w4.context_lens[b] > 8 * 256                    # decoded token never in a shared block
        assert np.array_equal(w4.block_tables[b, :8], w4.shared_blocks)
    others = np.setdiff1d(np.arange(256), w4.shared_seqs)
    own = np.concatenate([w4.block_tables[b][w4.block_tables[b] >= 0] for b in others] +
                         [w4.block_tables[b, 8:][w4.block_tables[b, 8:] >= 0] for b in w4.shared_seqs])
    assert len(np.unique(own)) == len(own) and not np.intersect1d(own, w4.shared_blocks).size
    # decode writes go to the last logical position, inside the sequence's own (unshared) blocks
    sm = w4.slot_mapping
    assert len(np.unique(sm)) == 256
    assert not np.isin(sm // 256, w4.shared_blocks).any()
    assert w4.kv_bytes(unique=False) - w4.kv_bytes(unique=True) == 63 * 2048 * 4096


def test_prefix_prefill_workload():
    w = wl.prefix_prefill_8b(seed=0)
    assert w.num_q_tokens == 32768 and list(w.cu_seqlens_q[:3]) == [0, 2048, 4096]
    assert w.cu_seqlens_k[-1] == 16 * 4096
    assert np.all(w.block_tables[:, :8] == w.shared_blocks)
    assert w.positions.min() == 2048 and w.positions.max() == 4095
    assert not np.isin(w.slot_mapping // 256, w.shared_blocks).any()
    assert len(np.unique(w.slot_mapping)) == 32768
    assert abs(w.flops - 1.650e12) / 1.650e12 < 2e-3


def test_bf16_bits_rne():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -0.0, np.inf, np.nan], dtype=np.float32)
    assert list(wl.bf16_bits(x)) == [0x3F80, 0x3F80, 0x3F82, 0x8000, 0x7F80, 0x7FC0]
    np.testing.assert_array_equal(wl.bf16_to_f32(wl.bf16_bits(x[:5])),
                                  np.array([1.0, 1.0, 1.015625, -0.0, np.inf], np.float32))
