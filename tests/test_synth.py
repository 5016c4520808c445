"""The seeded input generators draw what the workload statements describe."""

import numpy as np

import kvsynth


def test_single_splice_workload():
    w = kvsynth.single_splice()
    assert w.capacity == 4096 and w.block_size == 4096 and w.n_blocks == 1
    assert w.directives.tolist() == [[1000, 1800, 16, 0]]


def test_batched_splice_draws():
    w = kvsynth.batched_splice()
    d = w.directives
    s_len = d[:, 1] - d[:, 0]
    assert w.n_seq == 64 and w.shape.n_layers == 61
    assert s_len.min() >= 64 and s_len.max() <= 8192
    assert d[:, 2].min() >= 8 and d[:, 2].max() <= 64
    assert (d[:, 1] <= w.seq_lens).all() and (d[:, 0] >= 0).all()
    assert len(np.unique(w.block_tables)) == w.block_tables.size
    assert np.array_equal(kvsynth.batched_splice().directives, d)


def test_gather_draws():
    w = kvsynth.registry_gather()
    assert len(w.lens) == 32 and w.lens.sum() <= 40960
    assert w.lens.min() >= 256 and w.lens.max() <= 2048
    assert w.base_pos.min() >= 0 and w.base_pos.max() <= 60000
    order = np.argsort(w.p_target)
    ends = w.p_target[order] + w.lens[order]
    assert (w.p_target[order][1:] >= ends[:-1]).all()
    assert ends[-1] <= 40960 and w.p_target.min() >= 0
    assert len(np.unique(w.block_table)) == 640 and w.block_table.max() < 1024


def test_gqa_patch_draws():
    w = kvsynth.gqa_patch()
    assert (w.base_pos >= 0).all()
    assert np.abs(w.deltas).max() <= 30000
    assert sorted(w.p_target.tolist()) == [30720 + 1024 * i for i in range(16)]
    assert w.dst_slots == 30720 + 16 * 1024


def test_decode_draws():
    w = kvsynth.rotate_on_read_decode()
    assert w.block_tables.shape == (32, 512) and w.pending_delta.shape == (32, 512)
    assert np.abs(w.pending_delta).max() <= 100000
    assert abs(w.scale - 1 / 24.0) < 1e-15


def test_normal_range_regenerates_any_slice_of_a_fill():
    """normal_range_ reproduces every element range of fill_normal_, across
    slab boundaries and in the ragged last slab (the full-size parity tests
    regenerate pre-splice contents this way instead of keeping a copy)."""
    import torch
    t = torch.empty(10_000, dtype=torch.bfloat16)
    kvsynth.fill_normal_(t, 3, 1, slab_elems=1024)
    for lo, n in [(0, 10000), (5, 17), (1000, 2000), (9000, 1000), (1023, 2), (9999, 1)]:
        out = torch.empty(n, dtype=torch.bfloat16)
        kvsynth.normal_range_(out, lo, 10000, 3, 1, slab_elems=1024)
        assert torch.equal(out, t[lo:lo + n]), (lo, n)
