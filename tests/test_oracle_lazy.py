"""Pins of oracle.lazy (block-table splice) against the eager splice's
per-slot map (oracle.splice.source_of, itself pinned by list slicing), block
conservation and the rotation composition it relies on."""

import numpy as np
import pytest

from oracle import lazy, rope, splice


def _draw(r, B, nblocks):
    bt = r.permutation(10 * nblocks)[:nblocks].astype(np.int64)
    pend = r.integers(-100000, 100000, size=nblocks, endpoint=True)
    return bt, pend


def _cases(seed=0, count=300):
    r = np.random.default_rng([20260601, 77, seed])
    for _ in range(count):
        B = int(r.choice([1, 2, 4, 64]))
        cap_b = int(r.integers(1, 40))
        n = int(r.integers(0, cap_b * B + 1))
        s0 = B * int(r.integers(0, n // B + 1))
        s1 = B * int(r.integers(s0 // B, n // B + 1))
        rl = B * int(r.integers(0, cap_b + 1))
        if n + rl - (s1 - s0) > cap_b * B:
            continue
        bt, pend = _draw(r, B, cap_b)
        stubs = 100000 + r.permutation(1000)[: rl // B]
        yield B, n, s0, s1, rl, bt, pend, stubs


def _check_slots(B, n, s0, s1, rl, bt, pend, stubs, out):
    new_bt, new_pend, freed, new_len = out
    p = splice.plan(n, s0, s1, rl, splice.AMORTIZE, len(bt) * B)
    assert new_len == p.new_len
    for x in range(new_len):
        kind, i = splice.source_of(p, x)
        phys = new_bt[x // B] * B + x % B
        if kind == "stub":
            assert phys == stubs[i // B] * B + i % B
            assert new_pend[x // B] == 0
        else:
            assert phys == bt[i // B] * B + i % B
            want = pend[i // B] + (p.delta if i >= s1 else 0)
            assert new_pend[x // B] == want


def test_lazy_tables_match_eager_slot_map():
    seen = 0
    for B, n, s0, s1, rl, bt, pend, stubs in _cases():
        out = lazy.lazy_splice_tables(bt, pend, n, s0, s1, rl, B, stubs)
        _check_slots(B, n, s0, s1, rl, bt, pend, stubs, out)
        seen += 1
    assert seen > 150


def test_lazy_blocks_conserved_and_tail_cleared():
    for B, n, s0, s1, rl, bt, pend, stubs in _cases(seed=1):
        new_bt, new_pend, freed, new_len = lazy.lazy_splice_tables(bt, pend, n, s0, s1, rl, B, stubs)
        nb_old, nb_new = -(-n // B), -(-new_len // B)
        live = list(new_bt[:nb_new]) + list(freed)
        assert sorted(live) == sorted(list(bt[:nb_old]) + list(stubs))
        assert list(freed) == list(bt[s0 // B:s1 // B])
        assert (new_bt[nb_new:nb_old] == -1).all() and (new_pend[nb_new:nb_old] == 0).all()
        assert (new_bt[max(nb_old, nb_new):] == bt[max(nb_old, nb_new):]).all()


def test_lazy_matches_worked_example_shape():
    """Block-aligned variant of the single-sequence example: 4096 slots in
    64-slot blocks, [1024, 1792) replaced by 64 slots: Delta = -704."""
    bt = np.arange(64) + 1000
    pend = np.zeros(64, np.int64)
    new_bt, new_pend, freed, new_len = lazy.lazy_splice_tables(bt, pend, 4096, 1024, 1792, 64, 64, [7])
    assert new_len == 4096 - 704
    assert list(freed) == list(range(1016, 1028))
    assert new_bt[16] == 7 and new_pend[16] == 0
    assert new_bt[17] == 1028 and new_pend[17] == -704
    assert new_bt[52] == 1063 and (new_bt[53:64] == -1).all()


def test_lazy_rejects_misaligned_and_overflow():
    bt, pend = np.arange(8), np.zeros(8, np.int64)
    with pytest.raises(ValueError):
        lazy.lazy_splice_tables(bt, pend, 32, 3, 8, 4, 4, [1])          # s_start not a block multiple
    with pytest.raises(ValueError):
        lazy.lazy_splice_tables(bt, pend, 32, 4, 8, 6, 4, [1, 2])       # |R| not a block multiple
    with pytest.raises(ValueError):
        lazy.lazy_splice_tables(bt, pend, 32, 0, 4, 8, 4, [1, 2])       # 36 slots > capacity 32


def test_lazy_negative_control_missing_shift_fails():
    """A mutant that re-indexes blocks but forgets to add Delta to the pending
    shift must fail the slot-map pin."""
    B, n, s0, s1, rl = 4, 40, 8, 20, 4
    r = np.random.default_rng(5)
    bt, pend = _draw(r, B, 12)
    stubs = [99]
    new_bt, new_pend, freed, new_len = lazy.lazy_splice_tables(bt, pend, n, s0, s1, rl, B, stubs)
    bad_pend = new_pend.copy()
    bad_pend[(s0 + rl) // B:-(-new_len // B)] -= (rl - (s1 - s0))
    with pytest.raises(AssertionError):
        _check_slots(B, n, s0, s1, rl, bt, pend, stubs, (new_bt, bad_pend, freed, new_len))


def test_pending_composition_is_one_rotation():
    """The attended key after a lazy splice is R(pend + Delta) of the stored
    key; that equals rotating twice (R(Delta) R(pend)) up to fp64 rounding."""
    r = np.random.default_rng(9)
    th = rope.inv_freq(64, 10000.0)
    k = r.standard_normal((50, 64))
    a = r.integers(-100000, 100000, size=50)
    d = -704
    once = rope.rotate(k, a + d, 1, 64, th)
    twice = rope.rotate(rope.rotate(k, a, 1, 64, th), np.full(50, d), 1, 64, th)
    assert np.abs(once - twice).max() < 1e-9
