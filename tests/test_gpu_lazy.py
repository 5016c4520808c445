"""Parity of leyline_splice_lazy and kv_relocate_gather_lazy (HIP, through
the C ABI): the edited block tables and pending shifts are compared integer
for integer with the oracle, and a rotate-on-read decode over the lazily
spliced or gathered cache with the fp64 oracle on the composed keys."""

import math

import numpy as np
import pytest

import kvsynth
from oracle import bf16 as ob, decode as odec, lazy as olazy, rope as orope, splice as osplice, tolerance

pytestmark = pytest.mark.gpu

TH = orope.inv_freq(64, 10000.0)


def _tables(seqs, bt_stride, B, n_blocks, keys):
    r = kvsynth.rng(21, *keys)
    perm = r.permutation(n_blocks).astype(np.int32)
    n = len(seqs)
    bt = perm[: n * bt_stride].reshape(n, bt_stride).copy()
    pend = r.integers(-100000, 100000, size=(n, bt_stride), endpoint=True).astype(np.int32)
    spare = perm[n * bt_stride:]
    return bt, pend, spare


def _apply(bt_d, pd_d, B, lens, dirs, stubs):
    import torch
    import rope_rotation_splice_amd as rrs
    st_t = torch.from_numpy(np.asarray(stubs, np.int32)).cuda() if len(stubs) else None
    new_lens, freed, st = rrs.leyline_splice_lazy(bt_d, pd_d, B, lens, dirs, st_t)
    torch.cuda.synchronize()
    assert rrs.device_errors() == 0
    return new_lens, freed.cpu().numpy(), st


def _oracle_all(bt, pend, B, lens, dirs, stubs):
    bt2, pd2, freed, out = bt.astype(np.int64).copy(), pend.astype(np.int64).copy(), [], []
    off = 0
    for b, (n, d) in enumerate(zip(lens, dirs)):
        if d[3] == osplice.FORGET:
            out.append(d[0])
            continue
        k = d[2] // B
        nb, npd, fr, nl = olazy.lazy_splice_tables(bt[b], pend[b], n, d[0], d[1], d[2], B, stubs[off:off + k])
        off += k
        bt2[b], pd2[b] = nb, npd
        freed += list(fr)
        out.append(nl)
    return bt2, pd2, np.array(freed, np.int64), np.array(out)


@pytest.mark.parametrize("B", [4, 64])
def test_lazy_tables_bit_exact(B):
    import torch
    bt_stride = 40
    seqs = [  # (N, s_start, s_end, r_len, mode) in blocks * B, plus tails
        (30 * B + (3 if B > 4 else 1), 5 * B, 9 * B, 2 * B, 0),      # shrink, partial last block
        (25 * B, 3 * B, 4 * B, 3 * B, 0),                           # growth
        (20 * B, 0, 20 * B, 0, 0),                                  # everything replaced by nothing
        (18 * B, 7 * B, 12 * B, B, 1),                              # FORGET: unchanged
        (10 * B, 10 * B, 10 * B, 30 * B, 0),                        # append at the end, fills capacity
        (12 * B, 4 * B, 4 * B, 0, 0),                               # empty range, no stub: identity
    ]
    bt, pend, spare = _tables(seqs, bt_stride, B, 6 * bt_stride + 64, keys=(B,))
    lens = [s[0] for s in seqs]
    dirs = [s[1:] for s in seqs]
    n_stub = sum(d[2] // B for d in dirs if d[3] == 0)
    stubs = spare[:n_stub]
    bt_d, pd_d = torch.from_numpy(bt.copy()).cuda(), torch.from_numpy(pend.copy()).cuda()
    new_lens, freed, st = _apply(bt_d, pd_d, B, lens, dirs, stubs)
    bt2, pd2, fr2, nl2 = _oracle_all(bt, pend, B, lens, dirs, stubs)
    assert st == 1                                                  # one FORGET in the batch
    assert list(new_lens) == list(nl2)
    assert (bt_d.cpu().numpy() == bt2).all()
    assert (pd_d.cpu().numpy() == pd2).all()
    assert list(freed) == list(fr2)


def test_lazy_shift_overflow_flagged():
    import torch
    import rope_rotation_splice_amd as rrs
    B = 64
    bt = np.arange(8, dtype=np.int32).reshape(1, 8)
    pend = np.full((1, 8), 2 ** 31 - 10, np.int32)
    bt_d, pd_d = torch.from_numpy(bt).cuda(), torch.from_numpy(pend).cuda()
    st_t = torch.tensor([100], dtype=torch.int32).cuda()
    rrs.leyline_splice_lazy(bt_d, pd_d, B, [4 * B], [(0, 0, B, 0)], st_t)   # +64 overflows int32
    torch.cuda.synchronize()
    assert rrs.device_errors() & 8
    assert (pd_d.cpu().numpy()[0, 1:5] == 2 ** 31 - 10).all()


def _decode_check(pool_h, pool_d, bt_d, pd_d, lens, qn, qr, scale):
    import torch
    import rope_rotation_splice_amd as rrs
    cache = rrs.KVCache.mla(pool_d)
    out, lse = rrs.mla_decode_rotate_on_read(qn[1], qr[1], cache, 0, bt_d, pd_d,
                                             torch.tensor(lens, dtype=torch.int32).cuda(), scale,
                                             max_seq_len=bt_d.shape[1] * 64)
    torch.cuda.synchronize()
    assert rrs.device_errors() == 0
    o = ob.to_f64(out.view(torch.int16).cpu().numpy().view(np.uint16))
    lse = lse.cpu().numpy().astype(np.float64)
    bt, pd = bt_d.cpu().numpy(), pd_d.cpu().numpy()
    for b, n in enumerate(lens):
        phys = osplice.physical_rows(np.arange(n), bt[b], 64)
        rows = pool_h[phys]
        kr = ob.to_f64(rows[:, 512:])
        d = odec.token_deltas(pd[b], n, 64)
        qrb = ob.to_f64(qr[0][b])
        o_ref, l_ref = odec.mla_decode(ob.to_f64(qn[0][b]), qrb, ob.to_f64(rows[:, :512]), kr, d, scale, TH)
        assert tolerance.decode_close(o[b], o_ref, lse[b], l_ref).all(), f"sequence {b}"


def test_lazy_splice_then_decode_composes():
    """Two successive lazy splices, each followed by a rotate-on-read decode
    checked against the oracle: the pending shift carries both splices'
    Deltas and the key is rotated once, on read."""
    import torch
    B, bt_stride, heads = 64, 48, 128
    seqs = [(30 * B + 17, 5 * B, 9 * B, 2 * B, 0), (25 * B, 3 * B, 4 * B, 3 * B, 0)]
    n_blocks = 2 * bt_stride + 32
    bt, pend, spare = _tables(seqs, bt_stride, B, n_blocks, keys=(3,))
    r = kvsynth.rng(21, 4)
    pool_h = kvsynth.bf16_normal(r, (n_blocks * 64, 576))
    qn_h = kvsynth.bf16_normal(r, (2, heads, 512))
    qr_h = kvsynth.bf16_normal(r, (2, heads, 64))
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    pool_d = dev(pool_h).reshape(1, n_blocks, 64, 576)
    qn, qr = (qn_h, dev(qn_h)), (qr_h, dev(qr_h))
    bt_d, pd_d = torch.from_numpy(bt.copy()).cuda(), torch.from_numpy(pend.copy()).cuda()
    scale = 1.0 / math.sqrt(576.0)
    lens = [s[0] for s in seqs]
    _decode_check(pool_h, pool_d, bt_d, pd_d, lens, qn, qr, scale)
    used = 0
    for step_dirs in ([s[1:] for s in seqs], [(2 * B, 6 * B, B, 0), (10 * B, 11 * B, 2 * B, 0)]):
        n_stub = sum(d[2] // B for d in step_dirs)
        stubs = spare[used:used + n_stub]
        used += n_stub
        bt_h, pd_h = bt_d.cpu().numpy(), pd_d.cpu().numpy()
        new_lens, freed, st = _apply(bt_d, pd_d, B, lens, step_dirs, stubs)
        bt2, pd2, fr2, nl2 = _oracle_all(bt_h, pd_h, B, lens, step_dirs, stubs)
        assert st == 0 and list(new_lens) == list(nl2)
        assert (bt_d.cpu().numpy() == bt2).all() and (pd_d.cpu().numpy() == pd2).all()
        lens = [int(x) for x in new_lens]
        _decode_check(pool_h, pool_d, bt_d, pd_d, lens, qn, qr, scale)


# ---- kv_relocate_gather_lazy ------------------------------------------------

def _lazy_gather_case(B, bt_stride, n_seq, keys):
    """Tables for n_seq sequences and entries kept in spare pool blocks, placed
    at distinct block-aligned targets (ragged lengths only where the entry
    ends its sequence's content), half of them with their own shifts."""
    r = kvsynth.rng(22, *keys)
    n_blocks = n_seq * bt_stride + 16 * bt_stride
    perm = r.permutation(n_blocks).astype(np.int32)
    bt = perm[: n_seq * bt_stride].reshape(n_seq, bt_stride).copy()
    pend = r.integers(-100000, 100000, size=(n_seq, bt_stride), endpoint=True).astype(np.int32)
    spare = list(perm[n_seq * bt_stride:])
    ents = []
    for s in range(n_seq):
        k = 0
        while True:
            k += int(r.integers(0, 4))
            nb = int(r.integers(1, 6))
            if k + nb > bt_stride:
                break
            last = k + nb + 4 > bt_stride
            length = nb * B - (int(r.integers(1, B)) if last and B > 1 else 0)
            blocks = np.array([spare.pop() for _ in range(nb)], np.int32)
            own = r.integers(-50000, 50000, size=nb).astype(np.int32) if r.integers(0, 2) else None
            ents.append((s, blocks, own, length, int(r.integers(0, 200000)), k * B))
            k += nb
            if last:
                break
    return bt, pend, ents, n_blocks


def _run_lazy_gather(bt_d, pd_d, B, ents):
    import torch
    import rope_rotation_splice_amd as rrs
    objs = [rrs.LazyEntry(s, torch.from_numpy(bl).cuda(), ln, base, p,
                          None if own is None else torch.from_numpy(own).cuda())
            for s, bl, own, ln, base, p in ents]
    replaced, st = rrs.kv_relocate_gather_lazy(bt_d, pd_d, B, objs)
    torch.cuda.synchronize()
    assert rrs.device_errors() == 0
    return replaced.cpu().numpy(), st


def _lazy_gather_oracle(bt, pend, B, ents):
    bt2, pd2, rep = bt.astype(np.int64).copy(), pend.astype(np.int64).copy(), []
    for s in range(bt.shape[0]):
        mine = [(bl, own, ln, base, p) for (q, bl, own, ln, base, p) in ents if q == s]
        bt2[s], pd2[s], _ = olazy.lazy_gather_tables(bt[s], pend[s], B, mine)
    for s, bl, own, ln, base, p in ents:                 # replaced ids in entry order
        rep += list(bt[s][p // B: p // B + len(bl)])
    return bt2, pd2, np.array(rep, np.int64)


@pytest.mark.parametrize("B", [1, 16, 64])
def test_lazy_gather_tables_bit_exact(B):
    import torch
    bt, pend, ents, _ = _lazy_gather_case(B, 48, 5, keys=(B,))
    assert len(ents) > 10
    bt_d, pd_d = torch.from_numpy(bt.copy()).cuda(), torch.from_numpy(pend.copy()).cuda()
    rep, st = _run_lazy_gather(bt_d, pd_d, B, ents)
    bt2, pd2, rep2 = _lazy_gather_oracle(bt, pend, B, ents)
    assert st == 0
    assert (bt_d.cpu().numpy() == bt2).all() and (pd_d.cpu().numpy() == pd2).all()
    assert list(rep) == list(rep2)


def test_lazy_gather_many_entries_span_launches():
    """More entries than one launch carries (80), across 3 sequences."""
    import torch
    B, bt_stride = 4, 400
    r = kvsynth.rng(22, 9)
    bt = r.permutation(3 * bt_stride).astype(np.int32).reshape(3, bt_stride)
    pend = np.zeros_like(bt)
    ents, nxt = [], 10000
    for s in range(3):
        for k in range(0, bt_stride - 2, 3):
            ents.append((s, np.array([nxt, nxt + 1], np.int32), None, 2 * B, k * B + 7 * s, k * B))
            nxt += 2
    bt_d, pd_d = torch.from_numpy(bt.copy()).cuda(), torch.from_numpy(pend.copy()).cuda()
    rep, st = _run_lazy_gather(bt_d, pd_d, B, ents)
    bt2, pd2, rep2 = _lazy_gather_oracle(bt, pend, B, ents)
    assert len(ents) > 200 and st == 0
    assert (bt_d.cpu().numpy() == bt2).all() and (pd_d.cpu().numpy() == pd2).all()
    assert list(rep) == list(rep2)


def test_lazy_gather_shift_overflow_flagged():
    import torch
    import rope_rotation_splice_amd as rrs
    B = 64
    bt_d = torch.arange(8, dtype=torch.int32).reshape(1, 8).cuda()
    pd_d = torch.zeros((1, 8), dtype=torch.int32).cuda()
    own = torch.full((2,), 2 ** 31 - 10, dtype=torch.int32).cuda()
    blocks = torch.tensor([70, 71], dtype=torch.int32).cuda()
    rrs.kv_relocate_gather_lazy(bt_d, pd_d, B, [rrs.LazyEntry(0, blocks, 2 * B, 0, 3 * B, own)])   # +192 overflows
    torch.cuda.synchronize()
    assert rrs.device_errors() & 8
    assert (pd_d.cpu().numpy()[0, 3:5] == 2 ** 31 - 10).all()
    assert (bt_d.cpu().numpy()[0, 3:5] == [70, 71]).all()


def test_lazy_gather_then_decode():
    """Registry entries placed by reference, then a rotate-on-read decode over
    the shared blocks checked against the fp64 oracle: the keys are attended
    at R(own shift + p_target - base_pos), applied once, on read."""
    import torch
    B, bt_stride, heads = 64, 48, 128
    bt, pend, ents, n_blocks = _lazy_gather_case(B, bt_stride, 3, keys=(5,))
    r = kvsynth.rng(22, 6)
    pool_h = kvsynth.bf16_normal(r, (n_blocks * 64, 576))
    qn_h = kvsynth.bf16_normal(r, (3, heads, 512))
    qr_h = kvsynth.bf16_normal(r, (3, heads, 64))
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    pool_d = dev(pool_h).reshape(1, n_blocks, 64, 576)
    bt_d, pd_d = torch.from_numpy(bt.copy()).cuda(), torch.from_numpy(pend.copy()).cuda()
    _run_lazy_gather(bt_d, pd_d, B, ents)
    # each sequence ends where its last entry ends (a ragged entry comes last)
    lens = [max([p + ln for (q, bl, own, ln, base, p) in ents if q == s] + [B]) for s in range(3)]
    _decode_check(pool_h, pool_d, bt_d, pd_d, lens, (qn_h, dev(qn_h)), (qr_h, dev(qr_h)), 1.0 / math.sqrt(576.0))


def test_lazy_splice_workload_full_size():
    """The lazy-splice benchmark's configuration (64 sequences x 32768 slots,
    512-entry tables, the batched-splice directives widened to blocks), table
    for table against the oracle."""
    import torch
    import bench
    wl = bench.SpliceLazy()
    w, B = wl.w, wl.w.block_size
    bt = w.block_tables.astype(np.int32)
    pend = kvsynth.rng(23, 1).integers(-100000, 100000, size=bt.shape, endpoint=True).astype(np.int32)
    n_stub = sum(d[2] // B for d in wl.dirs)
    stubs = np.arange(w.n_blocks, w.n_blocks + n_stub, dtype=np.int32)
    bt_d, pd_d = torch.from_numpy(bt.copy()).cuda(), torch.from_numpy(pend.copy()).cuda()
    lens = [int(x) for x in w.seq_lens]
    new_lens, freed, st = _apply(bt_d, pd_d, B, lens, wl.dirs, stubs)
    bt2, pd2, fr2, nl2 = _oracle_all(bt, pend, B, lens, wl.dirs, stubs)
    assert st == 0 and list(new_lens) == list(nl2)
    assert (bt_d.cpu().numpy() == bt2).all() and (pd_d.cpu().numpy() == pd2).all()
    assert list(freed) == list(fr2)


def test_lazy_gather_workload_full_size():
    """The lazy-gather benchmark's configuration (32 registry entries packed at
    block-aligned targets of one 590-block sequence) against the oracle."""
    import torch
    import bench
    wl = bench.GatherLazy()
    B = wl.w.block_size
    r = kvsynth.rng(23, 2)
    bt = r.permutation(4 * wl.bt_stride)[: wl.bt_stride].astype(np.int32).reshape(1, -1)
    pend = r.integers(-100000, 100000, size=bt.shape, endpoint=True).astype(np.int32)
    ents, nxt = [], 10 * wl.bt_stride
    for c in range(len(wl.nb)):
        n = int(wl.nb[c])
        own = r.integers(-5000, 5000, size=n).astype(np.int32) if c % 3 == 0 else None
        ents.append((0, np.arange(nxt, nxt + n, dtype=np.int32), own, n * B, int(wl.w.base_pos[c]), int(wl.tgt[c])))
        nxt += n
    bt_d, pd_d = torch.from_numpy(bt.copy()).cuda(), torch.from_numpy(pend.copy()).cuda()
    rep, st = _run_lazy_gather(bt_d, pd_d, B, ents)
    bt2, pd2, rep2 = _lazy_gather_oracle(bt, pend, B, ents)
    assert st == 0
    assert (bt_d.cpu().numpy() == bt2).all() and (pd_d.cpu().numpy() == pd2).all()
    assert list(rep) == list(rep2)


def test_lazy_gather_packed_batch_matches_the_oracle_twice():
    """A LazyBatch (entries packed once) gives the oracle's tables, and the
    same batch placed again on fresh tables gives them again."""
    import torch
    import rope_rotation_splice_amd as rrs
    B, bt_stride, n_seq = 16, 24, 3
    bt, pend, ents, _ = _lazy_gather_case(B, bt_stride, n_seq, (41,))
    want_bt, want_pd, want_rep = _lazy_gather_oracle(bt, pend, B, ents)
    objs = [rrs.LazyEntry(s, torch.from_numpy(bl).cuda(), ln, base, p,
                          None if own is None else torch.from_numpy(own).cuda())
            for s, bl, own, ln, base, p in ents]
    batch = rrs.LazyBatch(objs)
    for _ in range(2):
        bt_d, pd_d = torch.from_numpy(bt.copy()).cuda(), torch.from_numpy(pend.copy()).cuda()
        replaced, st = rrs.kv_relocate_gather_lazy(bt_d, pd_d, B, batch)
        torch.cuda.synchronize()
        assert st == 0 and rrs.device_errors() == 0
        assert np.array_equal(bt_d.cpu().numpy(), want_bt)
        assert np.array_equal(pd_d.cpu().numpy(), want_pd)
        assert np.array_equal(replaced.cpu().numpy(), want_rep)
