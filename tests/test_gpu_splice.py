"""Parity of leyline_splice (HIP, through the C ABI) against the fp64 oracle."""

import numpy as np
import pytest

import kvsynth
from oracle import bf16, rope as orope
from tests import relocation_cases as rc

pytestmark = pytest.mark.gpu


def _run(lay, n_layers, block_size, bps, seqs, keys, stubs_on=True, special=False, spare=3, rounds=1):
    """seqs: list of (N, s_start, s_end, r_len, mode).  Builds a paged pool with
    random block tables and spare canary blocks, splices, checks everything."""
    import torch
    import rope_rotation_splice_amd as rrs
    n_seq = len(seqs)
    n_blocks = n_seq * bps + spare
    r = kvsynth.rng(*keys, 99)
    perm = r.permutation(n_blocks).astype(np.int32)
    bt = perm[: n_seq * bps].reshape(n_seq, bps)
    pf, rp = rc.random_image(lay, n_layers, n_blocks * block_size, keys, special=special)
    # canary blocks: recognisable NaN payloads
    for blk in perm[n_seq * bps:]:
        pf[:, blk * block_size:(blk + 1) * block_size] = rc.SENTINEL
    cache, keep = rc.to_device(lay, pf, rp, n_blocks, block_size)
    d_bt = torch.from_numpy(bt).cuda()
    lens = [s[0] for s in seqs]
    dirs = [s[1:] for s in seqs]
    stubs_h, stubs_d = None, None
    if stubs_on:
        stubs_h, stubs_d = [], []
        for i, (n, s0, s1, rl, m) in enumerate(seqs):
            spf, srp = rc.random_image(lay, n_layers, rl, keys + (500 + i,))
            stubs_h.append((spf, srp))
            tp, tr = rc.rows_to_device(lay, spf, srp)
            stubs_d.append(rrs.Rows(tp, tr))
    before = (pf, rp)
    new_lens, st = rrs.leyline_splice(cache, d_bt, lens, dirs, stubs_d)
    torch.cuda.synchronize()
    after = rc.from_device(lay, cache)
    assert rrs.device_errors() == 0
    want = rc.check_splice(lay, before, after, bt, block_size, lens, dirs, stubs_h)
    assert list(new_lens) == want
    has_forget = any(s[4] == 1 for s in seqs)
    assert st == (rrs.KVR_FORGET_NEEDS_PREFILL if has_forget else 0)
    return cache, keep


DELTAS = [-1, -2, -63, -64, -65, -127, -129, -700, 1, 2, 63, 64, 65, 130, 0]


@pytest.mark.parametrize("block_size", [1, 4, 64])
@pytest.mark.parametrize("delta", DELTAS)
def test_splice_delta_sweep_mla(block_size, delta):
    cap = 1024
    bps = cap // block_size
    seqs = []
    # several sequences with ragged lengths and the same Delta
    for i, n in enumerate([1000, 777, 1021]):
        n = min(n, cap - max(delta, 0))
        s_len = 40 + 13 * i
        r_len = s_len + delta
        if r_len < 0:
            s_len, r_len = -delta, 0
        s0 = min(100 + 37 * i, n - s_len)
        seqs.append((n, s0, s0 + s_len, r_len, 0))
    _run(rc.MLA, 2, block_size, bps, seqs, (block_size, delta + 1000))


def test_splice_gqa_layout():
    seqs = [(900, 10, 300, 17, 0), (1024 - 40, 500, 510, 50, 0), (513, 0, 513, 5, 0)]
    _run(rc.GQA, 2, 16, 64, seqs, (77,))


def test_splice_fp32_keys():
    seqs = [(1000, 100, 400, 9, 0), (700, 699, 700, 60, 0)]
    _run(rc.MLA_F32, 3, 8, 128, seqs, (78,))


def test_splice_special_bit_patterns_and_no_stub():
    seqs = [(1000, 3, 900, 1, 0), (512, 200, 201, 40, 0)]
    _run(rc.MLA, 2, 64, 16, seqs, (79,), stubs_on=False, special=True)


def test_splice_forget_and_identity_in_batch():
    seqs = [(1000, 100, 200, 7, 1),          # FORGET: nothing moves, new_len = 100
            (800, 300, 340, 40, 0),          # Delta = 0: only the stub is written
            (900, 0, 0, 0, 0),               # empty directive
            (600, 599, 600, 1, 0),           # replace the last slot
            (1024 - 64, 960 - 64, 960 - 64, 64, 0)]   # pure insertion at the end
    _run(rc.MLA, 2, 64, 16, seqs, (80,))


def test_splice_many_sequences_multiple_launches():
    r = kvsynth.rng(81)
    seqs = []
    for i in range(37):                      # more sequences than one launch holds
        n = int(r.integers(300, 512))
        s_len = int(r.integers(0, 200))
        s0 = int(r.integers(0, n - s_len + 1))
        rl = int(r.integers(0, 40))
        if n + rl - s_len > 512:
            rl = 512 - n + s_len
        seqs.append((n, s0, s0 + s_len, rl, 0))
    _run(rc.MLA, 2, 64, 8, seqs, (81,))


def test_splice_back_to_back_reuses_workspace():
    """Two splices in a row on the same workspace: counters must come back zeroed."""
    seqs = [(1000, 100, 600, 3, 0), (1000, 10, 20, 30, 0)]
    for k in range(3):
        _run(rc.MLA, 2, 64, 16, seqs, (82, k))


def test_single_sequence_workload_with_drift():
    """The single-sequence workload: 4096 contiguous slots, [1000, 1800) -> 16
    stub slots, Delta = -784.  Keys are stored pre-rotated at their slot
    (bf16 of R(p) k_raw); after the splice every moved key is checked against
    the oracle and, for drift, against R(new slot) k_raw from scratch."""
    import torch
    import rope_rotation_splice_amd as rrs
    w = kvsynth.single_splice()
    lay = rc.MLA
    th = lay.theta()
    r = kvsynth.rng(1, 1)
    k_raw = r.standard_normal((4096, 64))
    stored = bf16.round_rne(orope.rotate(k_raw, np.arange(4096), 1, 64, th))
    pf = kvsynth.bf16_normal(r, (1, 4096, 512))
    rp = stored[None]
    cache, keep = rc.to_device(lay, pf, rp, 1, 4096)
    spf, srp = rc.random_image(lay, 1, 16, (1, 2))
    tp, tr = rc.rows_to_device(lay, spf, srp)
    d_bt = torch.zeros((1, 1), dtype=torch.int32, device="cuda")
    dirs = [tuple(int(x) for x in w.directives[0])]
    new_lens, st = rrs.leyline_splice(cache, d_bt, [4096], dirs, [rrs.Rows(tp, tr)])
    torch.cuda.synchronize()
    assert list(new_lens) == [3312] and st == 0
    after = rc.from_device(lay, cache)
    assert rrs.device_errors() == 0
    rc.check_splice(lay, (pf, rp), after, np.zeros((1, 1), np.int32), 4096, [4096], dirs, [(spf, srp)])
    got = bf16.to_f64(after[1][0, 1016:3312])
    scratch = orope.rotate(k_raw[1800:4096], np.arange(1016, 3312), 1, 64, th)
    rel = np.linalg.norm(got - scratch) / np.linalg.norm(scratch)
    assert rel <= 4.7e-3, rel
