"""Pins of oracle.lazy: the block-table splice against the eager splice's
per-slot map (oracle.splice.source_of, itself pinned by list slicing), block
conservation and the rotation composition it relies on; the block-table
gather against the slot each entry row must land in and against decoding
the eagerly relocated rows (oracle.gather + oracle.decode)."""

import numpy as np
import pytest

from oracle import decode, gather, lazy, rope, splice


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


# ---- lazy gather (registry entries placed by reference) -------------------

def _gather_case(r, B, cap_b):
    """A table with random ids and shifts, and up to three entries placed at
    distinct block-aligned targets (some ragged, some with their own pending
    shifts)."""
    bt, pend = _draw(r, B, cap_b)
    free = list(r.permutation(cap_b))
    placements, next_id = [], 50000
    for _ in range(int(r.integers(0, 4))):
        length = int(r.integers(0, 3 * B + 1))
        nb = -(-length // B)
        starts = [k for k in free if all(k + j in free for j in range(nb)) and k + nb <= cap_b]
        if not starts:
            continue
        k0 = int(r.choice(starts))
        for j in range(nb):
            free.remove(k0 + j)
        blocks = np.arange(next_id, next_id + nb)
        next_id += nb
        epend = None if r.integers(0, 2) else r.integers(-5000, 5000, size=nb)
        placements.append((blocks, epend, length, int(r.integers(0, 60000)), k0 * B))
    return bt, pend, placements


def test_lazy_gather_slot_map_and_replaced_ids():
    r = np.random.default_rng([20260601, 78])
    seen = 0
    for _ in range(300):
        B = int(r.choice([1, 2, 4, 64]))
        cap_b = int(r.integers(1, 24))
        bt, pend, pl = _gather_case(r, B, cap_b)
        new_bt, new_pend, replaced = lazy.lazy_gather_tables(bt, pend, B, pl)
        covered = {}
        rep = []
        for e, (blocks, epend, length, base, p) in enumerate(pl):
            for k in range(-(-length // B)):
                covered[p // B + k] = (e, k)
                rep.append(bt[p // B + k])
            for x in range(p, p + length):              # every slot of the entry
                row = x - p
                assert new_bt[x // B] * B + x % B == blocks[row // B] * B + row % B
                owed = 0 if epend is None else epend[row // B]
                # the key at slot x is the entry's key for position base + row,
                # stored rotated to base + row - owed: it owes x - (base + row - owed)
                assert new_pend[x // B] == x - (base + row - owed)
        for k in range(cap_b):
            if k not in covered:
                assert new_bt[k] == bt[k] and new_pend[k] == pend[k]
        assert list(replaced) == rep
        seen += len(pl)
    assert seen > 200


def test_lazy_gather_rejects():
    bt, pend = np.arange(8), np.zeros(8, np.int64)
    with pytest.raises(ValueError):
        lazy.lazy_gather_tables(bt, pend, 4, [([1], None, 4, 0, 2)])                    # target off a block edge
    with pytest.raises(ValueError):
        lazy.lazy_gather_tables(bt, pend, 4, [([1, 2], None, 8, 0, 28)])                # past the table
    with pytest.raises(ValueError):
        lazy.lazy_gather_tables(bt, pend, 4, [([1], None, 8, 0, 0)])                    # too few blocks
    with pytest.raises(ValueError):
        lazy.lazy_gather_tables(bt, pend, 4, [([1], None, 3, 0, 4), ([2], None, 2, 9, 4)])   # shared block


def test_lazy_gather_then_decode_equals_eager_gather():
    """Decoding through the lazily edited tables (keys rotated on read by
    their pending shifts) gives what decoding the eagerly relocated rows
    gives (keys rotated by R(p_target - base_pos) when moved, shift 0), and a
    table that forgets the entry's own pending shift does not."""
    r = np.random.default_rng(31)
    B, cap_b, H, Dc, Dr = 4, 12, 2, 8, 8
    th = rope.inv_freq(Dr, 10000.0)
    n_pool = 40
    pool_c, pool_r = r.standard_normal((n_pool * B, Dc)), r.standard_normal((n_pool * B, Dr))
    bt = r.permutation(20)[:cap_b].astype(np.int64)
    pend = r.integers(-3000, 3000, size=cap_b)
    # two entries living in pool blocks 30.. with own shifts; the second is
    # ragged and ends the sequence (rows past an entry inside its last block
    # are the entry block's, so a ragged entry can only come last)
    ents = [(np.array([30, 31]), np.array([7, -11]), 8, 1000, 2 * B),
            (np.array([33, 34, 35]), None, 10, 52000, 7 * B)]
    N = 7 * B + 10
    new_bt, new_pend, _ = lazy.lazy_gather_tables(bt, pend, B, ents)
    qn, qr = r.standard_normal((H, Dc)), r.standard_normal((H, Dr))

    def lazy_side(tab_bt, tab_pend):
        phys = np.array([tab_bt[x // B] * B + x % B for x in range(N)])
        return decode.mla_decode(qn, qr, pool_c[phys], pool_r[phys], decode.token_deltas(tab_pend, N, B), 0.3, th)

    # eager: rows copied to the slots, keys rotated on the move, shift 0
    ckv, kr, dtok = np.zeros((N, Dc)), np.zeros((N, Dr)), np.zeros(N, np.int64)
    for x in range(N):
        ckv[x], kr[x], dtok[x] = pool_c[bt[x // B] * B + x % B], pool_r[bt[x // B] * B + x % B], pend[x // B]
    for blocks, epend, length, base, p in ents:
        for row in range(length):
            src = blocks[row // B] * B + row % B
            owed = 0 if epend is None else epend[row // B]
            ckv[p + row] = pool_c[src]
            kr[p + row] = rope.rotate(pool_r[src][None], owed + gather.chunk_delta(p, base), 1, Dr, th)[0]
            dtok[p + row] = 0
    o_e, l_e = decode.mla_decode(qn, qr, ckv, kr, dtok, 0.3, th)
    o_l, l_l = lazy_side(new_bt, new_pend)
    assert np.abs(o_l - o_e).max() < 1e-10 and np.abs(l_l - l_e).max() < 1e-10
    bad = new_pend.copy()
    bad[2:4] -= np.array([7, -11])                       # entry shift forgotten
    o_b, _ = lazy_side(new_bt, bad)
    assert np.abs(o_b - o_e).max() > 1e-6
