"""Pins of the splice oracle: brute-force index maps, closure from scratch,
golden figures of the single-sequence workload, error conventions."""

import json
import os

import numpy as np
import pytest

from oracle import bf16, rope, splice

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
DIM, BASE = 64, 10000.0
TH = rope.inv_freq(DIM, BASE)


def test_golden_single_sequence_plan():
    g = json.load(open(os.path.join(GOLDEN, "single_splice.json")))
    p = splice.plan(g["n"], g["s_start"], g["s_end"], g["r_len"], splice.AMORTIZE, capacity=g["n"])
    assert p.delta == g["delta"]
    assert p.moved_rows == g["moved_rows"]
    assert p.new_len == g["new_len"]


def _rows_with_ids(n, tag):
    """pf rows carrying a unique id (tag * 1000 + slot) in their first two words."""
    ids = np.arange(n, dtype=np.int64) + tag * 1000
    pf = np.zeros((n, 4), np.uint16)
    pf[:, 0] = ids & 0xFFFF
    pf[:, 1] = ids >> 16
    return pf


def _ids(pf):
    return (pf[:, 0].astype(np.int64) | (pf[:, 1].astype(np.int64) << 16)).tolist()


def test_index_map_brute_force_against_list_slicing():
    """Every directive on N <= 10 (all s <= e <= N, |R| <= 4): the content map
    read back from the rows equals old[:s] + stub + old[e:N]."""
    r = np.random.default_rng(0)
    count = 0
    for n in range(0, 11):
        pf = _rows_with_ids(n, 1)
        rw = bf16.round_rne(r.standard_normal((n, DIM)))
        for s in range(n + 1):
            for e in range(s, n + 1):
                for rl in range(5):
                    stub = _rows_with_ids(rl, 2)
                    stub_r = bf16.round_rne(r.standard_normal((rl, DIM)))
                    p = splice.plan(n, s, e, rl, splice.AMORTIZE)
                    ex = splice.splice_sequence(p, pf, rw, stub, stub_r, 1, DIM, TH)
                    old = _ids(pf)
                    assert _ids(ex.pf_bits) == old[:s] + _ids(stub) + old[e:n]
                    assert p.new_len == len(old[:s]) + rl + len(old[e:n])
                    # rotated exactly the rows that came from downstream, when they moved
                    moved = np.array([False] * s + [False] * rl + [p.delta != 0] * (n - e), bool)
                    assert np.array_equal(ex.rotated, moved)
                    # non-rotated rotary rows are bit-exact copies
                    keep = ~ex.rotated
                    src_r = np.concatenate([rw[:s], stub_r, rw[e:n]])
                    assert np.array_equal(ex.rope_bits[keep], src_r[keep])
                    count += 1
    assert count > 1000


def test_rotated_rows_equal_rope_from_scratch_at_new_slot():
    """Keys stored pre-rotated at their slot i (exact float64 values) come out as
    the key rotated from scratch at its new slot: R(Delta) R(i) k = R(i + Delta) k
    (Leyline §2.2).  A wrong sign of Delta or a wrong destination fails here."""
    r = np.random.default_rng(1)
    n = 300
    k_raw = r.standard_normal((n, DIM))
    stored = rope.rotate(k_raw, np.arange(n), 1, DIM, TH)
    for (s, e, rl) in [(100, 180, 16), (10, 12, 40), (0, 300, 5), (250, 250, 3), (40, 140, 100)]:
        p = splice.plan(n, s, e, rl, splice.AMORTIZE)
        # feed float32 words so that the stored values are kept (nearly) exact
        words = stored.astype(np.float32)
        ex = splice.splice_sequence(p, np.zeros((n, 2), np.uint16), words, None, None, 1, DIM, TH,
                                    rope_is_bf16=False)
        for x in range(p.new_len):
            if s <= x < s + rl:
                continue
            src = x if x < s else x - p.delta
            scratch = rope.rotate(k_raw[src], x, 1, DIM, TH)
            # tolerance: float32 storage of the pre-rotated key
            assert np.max(np.abs(ex.rope_ref[x] - scratch)) <= 1e-6 * np.linalg.norm(k_raw[src])


def test_forget_moves_nothing():
    p = splice.plan(500, 100, 200, 7, splice.FORGET)
    assert p.new_len == 100 and p.moved_rows == 0 and p.delta == 0
    with pytest.raises(ValueError):
        splice.splice_sequence(p, np.zeros((500, 2), np.uint16), np.zeros((500, DIM), np.uint16),
                               None, None, 1, DIM, TH)


@pytest.mark.parametrize("args", [(10, 5, 4, 1), (10, -1, 4, 1), (10, 3, 11, 1), (10, 3, 4, -1)])
def test_malformed_directives_rejected(args):
    with pytest.raises(ValueError):
        splice.plan(*args)


def test_capacity_checked_on_growth():
    splice.plan(60, 10, 12, 6, capacity=64)
    with pytest.raises(ValueError):
        splice.plan(60, 10, 12, 7, capacity=64)


def test_delta_zero_is_identity_bit_exact():
    r = np.random.default_rng(2)
    n = 50
    pf = r.integers(0, 65535, size=(n, 8)).astype(np.uint16)
    rw = r.integers(0, 65535, size=(n, DIM)).astype(np.uint16)     # includes NaN/-0 patterns
    stub = r.integers(0, 65535, size=(5, 8)).astype(np.uint16)
    stub_r = r.integers(0, 65535, size=(5, DIM)).astype(np.uint16)
    p = splice.plan(n, 10, 15, 5)
    ex = splice.splice_sequence(p, pf, rw, stub, stub_r, 1, DIM, TH)
    assert not ex.rotated.any()
    want_pf = np.concatenate([pf[:10], stub, pf[15:]])
    want_r = np.concatenate([rw[:10], stub_r, rw[15:]])
    assert np.array_equal(ex.pf_bits, want_pf)
    assert np.array_equal(ex.rope_bits, want_r)


def test_paged_translation_brute_force():
    r = np.random.default_rng(3)
    for bsz in (1, 4, 64):
        nb = 12
        bt = r.permutation(nb + 5)[:nb]
        table = {}
        for lb in range(nb):
            for o in range(bsz):
                table[lb * bsz + o] = int(bt[lb]) * bsz + o
        slots = np.arange(nb * bsz)
        got = splice.physical_rows(slots, bt, bsz)
        assert got.tolist() == [table[int(x)] for x in slots]
