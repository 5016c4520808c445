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


@pytest.mark.parametrize("delta", [-4096, -8184, 4096])
def test_splice_shifts_of_the_batched_workload(delta):
    """Shifts as large as the batched workload draws (|Delta| up to 8184),
    on two layers with 16K-slot sequences."""
    cap, B = 16384, 64
    seqs = []
    for i, n in enumerate([16000, 12345]):
        n = min(n, cap - max(delta, 0))
        s_len = (-delta if delta < 0 else 0) + 40 + 9 * i
        r_len = s_len + delta
        s0 = 300 + 77 * i
        seqs.append((n, s0, s0 + s_len, r_len, 0))
    _run(rc.MLA, 2, B, cap // B, seqs, (B, delta + 10000))


@pytest.mark.parametrize("block_size", [16, 64])
@pytest.mark.parametrize("delta", [-3000, -700, 700, 3000])
def test_splice_large_call_and_small_call_paths(block_size, delta):
    """The same directives as one call of four layers (over 65,536 moved
    rows in all: the ticketed mover streams it) and as a one-layer call (few
    rows: chain tiles of the band mover), both checked against the oracle."""
    cap = 12288
    seqs = []
    for i, n in enumerate([12000, 9999, 11111]):
        n = min(n, cap - max(delta, 0))
        s_len = max(0, -delta) + 30 + 11 * i
        r_len = s_len + delta
        s0 = 200 + 91 * i
        seqs.append((n, s0, s0 + s_len, r_len, 0))
    moved = sum(n - s1 for n, s0, s1, r, m in seqs)
    assert moved * 4 >= 65536 > moved
    for layers in (4, 1):
        _run(rc.MLA, layers, block_size, cap // block_size, seqs, (block_size, delta + 20000, layers))


@pytest.mark.parametrize("delta", [-65536, 65536, -100000, 100000])
def test_splice_large_shifts(delta):
    """|Delta| of 2^16 and 1e5 on one layer: the rotation angle Delta*theta_j
    must be reduced in double precision (an fp32 angle at 1e5 rad is off by
    ~4e-3 rad, far outside the 1-ulp bar).  Growth takes a stub of |R| =
    |S| + Delta rows; a shrink replaces |S| = |R| - Delta rows."""
    B = 64
    if delta < 0:
        s_len, r_len = -delta + 31, 31
        n = s_len + 3000 + 17
    else:
        s_len, r_len = 13, 13 + delta
        n = 2900
    cap = -(-(max(n, n + delta)) // B) * B
    seqs = [(n, 1000, 1000 + s_len, r_len, 0)]
    _run(rc.MLA, 1, B, cap // B, seqs, (B, abs(delta) % 9973, delta > 0))


@pytest.mark.parametrize("delta", [-1, -30, -700, 2, 25, 130])
def test_splice_block_size_not_a_power_of_two(delta):
    # 24-row blocks: the kernels divide slots by the block size instead of shifting
    cap = 24 * 43
    seqs = []
    for i, n in enumerate([1000, 801, 977]):
        n = min(n, cap - max(delta, 0))
        s_len = 50 + 7 * i
        r_len = max(0, s_len + delta)
        s_len = r_len - delta
        s0 = min(90 + 31 * i, n - s_len)
        seqs.append((n, s0, s0 + s_len, r_len, 0))
    _run(rc.MLA, 2, 24, 43, seqs, (24, delta + 2000))


@pytest.mark.parametrize("layout", ["MLA", "GQA", "MLA_F32"])
@pytest.mark.parametrize("block_size", [1, 24, 64])
@pytest.mark.parametrize("delta", [-700, -1, 25, 130])
def test_splice_single_sequence_one_item_launch(layout, block_size, delta):
    """A small call with one sequence takes the band mover's one-item form:
    the item's scalars arrive as leading (preloaded) kernel arguments and its
    (cos, sin) table is formed on the host in float64.  Every layout (MLA
    bf16, GQA with 8 rotary heads, fp32 keys), a block size of 1, one that is
    not a power of two, and shrinks and growth (the stub rows that land on the
    chains' last sources) against the oracle."""
    lay = getattr(rc, layout)
    cap = 24 * 43 if block_size == 24 else 1024
    n = min(1000, cap - max(delta, 0))
    s_len = max(40, -delta + 3)
    r_len = s_len + delta
    s0 = 100
    _run(lay, 2, block_size, cap // block_size, [(n, s0, s0 + s_len, r_len, 0)],
         (block_size, delta + 3000, len(layout)))


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


def _check_every_slab(w, cfg):
    """Splice workload ``w`` (pool filled from seed keys (cfg, 1), stubs from
    (cfg, 2, b)) and check every (sequence, layer) slab.

    The pool is not copied before the splice: each layer's pre-splice
    contents are regenerated from their seeds on the device (the same seeded
    draws that filled the pool), one layer at a time.  Per slab, the oracle's
    splice (oracle.splice.splice_sequence on the slab's rotary column, with
    the oracle's slot map) gives the expected rotary words: prefix and stub
    bit-exact, moved keys within one bf16 ulp of R(Delta) x in fp64.  The
    position-free words of every new slot are compared bit for bit, on the
    device, with the old row (or stub row) the oracle's slot map names."""
    import concurrent.futures as cf
    import os
    import torch
    import rope_rotation_splice_amd as rrs
    from oracle import splice as osplice, tolerance
    L, B = w.shape.n_layers, w.block_size
    shape = (L, w.n_blocks, B, 576)
    total = int(np.prod(shape))
    per_layer = total // L
    pool = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    kvsynth.fill_normal_(pool, cfg, 1)
    cache = rrs.KVCache.mla(pool)
    bt = torch.from_numpy(w.block_tables).cuda()
    stubs_t, stubs = [], []
    for b in range(w.n_seq):
        st = torch.empty((L, int(w.directives[b, 2]), 576), dtype=torch.bfloat16, device="cuda")
        kvsynth.fill_normal_(st, cfg, 2, b)
        stubs_t.append(st)
        stubs.append(rrs.Rows(st[..., :512], st[..., 512:]))
    old = torch.empty((w.n_blocks * B, 576), dtype=torch.bfloat16, device="cuda")
    kvsynth.normal_range_(old, 0, total, cfg, 1)
    assert torch.equal(old.view(torch.int16), pool[0].reshape(-1, 576).view(torch.int16)), \
        "regenerating the seeded fill does not reproduce it"

    new_lens, st = rrs.leyline_splice(cache, bt, w.seq_lens.tolist(),
                                      [tuple(int(x) for x in d) for d in w.directives], stubs)
    torch.cuda.synchronize()
    assert st == 0 and rrs.device_errors() == 0
    th = orope.inv_freq(64, 10000.0)
    plans, maps = [], []
    for b in range(w.n_seq):
        d = w.directives[b]
        p = osplice.plan(int(w.seq_lens[b]), int(d[0]), int(d[1]), int(d[2]), int(d[3]))
        assert new_lens[b] == p.new_len
        is_stub, idx = osplice.sources(p, np.arange(p.new_len))
        phys_new = osplice.physical_rows(np.arange(p.new_len), w.block_tables[b], B)
        phys_old = osplice.physical_rows(np.arange(p.n), w.block_tables[b], B)
        src_old = osplice.physical_rows(idx[~is_stub], w.block_tables[b], B)
        plans.append(p)
        maps.append(tuple(torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in
                          (phys_new, phys_old, src_old, np.flatnonzero(~is_stub), np.flatnonzero(is_stub),
                           idx[is_stub])))
    h16 = lambda t: t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    def rope_check(b, l, old_rp, new_rp, stub_rp):
        p = plans[b]
        ex = osplice.splice_sequence(p, np.zeros((p.n, 0), np.uint16), old_rp, np.zeros((len(stub_rp), 0), np.uint16),
                                     stub_rp, 1, 64, th, rope_is_bf16=True)
        plain = ~ex.rotated
        bad = int((new_rp[plain] != ex.rope_bits[plain]).sum())
        ok = tolerance.bf16_close(new_rp[ex.rotated], ex.rope_ref[ex.rotated], ex.pair_norm[ex.rotated])
        return b, l, bad, int((~ok).sum()), int(ex.rotated.sum())

    checked, rotated = 0, 0
    failures = []

    def drain(fs):
        nonlocal checked, rotated
        for f in fs:
            b, l, bad, out, n_rot = f.result()
            checked += 1
            rotated += n_rot
            if bad or out:
                failures.append(f"seq {b} layer {l}: {bad} unrotated words differ, {out} rotated outside tolerance")

    with cf.ThreadPoolExecutor(max_workers=min(16, len(os.sched_getaffinity(0)))) as ex:
        futs = []
        for l in range(L):
            if l >= 2:                  # bound the host backlog to two layers of slabs
                drain(futs[:w.n_seq])
                futs = futs[w.n_seq:]
            if l:
                kvsynth.normal_range_(old, l * per_layer, total, cfg, 1)
            cur = pool[l].reshape(-1, 576)
            for b in range(w.n_seq):
                phys_new, phys_old, src_old, at_old, at_stub, stub_idx = maps[b]
                got = cur[phys_new]
                # position-free words of every new slot, bit for bit, on the device
                pf_ok = torch.equal(got[at_old, :512].view(torch.int16), old[src_old, :512].view(torch.int16))
                st_ok = torch.equal(got[at_stub, :512].view(torch.int16),
                                    stubs_t[b][l][stub_idx, :512].view(torch.int16))
                if not (pf_ok and st_ok):
                    failures.append(f"seq {b} layer {l}: position-free words differ")
                futs.append(ex.submit(rope_check, b, l, h16(old[phys_old, 512:]), h16(got[:, 512:]),
                                      h16(stubs_t[b][l][:, 512:])))
            print(f"layer {l}: {w.n_seq} slabs queued, {checked} checked", flush=True)
        drain(futs)
    print(f"checked {checked} (sequence, layer) slabs, {rotated} rotated rows", flush=True)
    assert checked == w.n_seq * L
    assert not failures, failures[:8]
    return checked


@pytest.mark.parametrize("layers", [3, 12])
def test_batched_splice_every_slab_small(layers):
    """The every-slab check on a small batched draw (growth allowed, so both
    shift directions), blocks of 16: three layers take the band mover, twelve
    the ticketed one."""
    w = kvsynth.batched_splice(n_seq=6, capacity=4096, n_layers=layers, block_size=16, s_range=(1, 700),
                               r_range=(0, 900), cfg=31, allow_growth=True)
    assert _check_every_slab(w, 31) == 6 * layers


@pytest.mark.timeout(900)
def test_batched_splice_full_workload_every_slab():
    """The batched-splice workload at full size (64 sequences x 32768 slots x
    61 layers, 64-row blocks, 147 GB resident), in the launch configuration
    the benchmark times: all 3904 (sequence, layer) slabs checked."""
    w = kvsynth.batched_splice()
    assert _check_every_slab(w, 3) == 64 * 61


def test_splice_after_decode_on_the_same_stream():
    """A decode's split partials must not land in the splice's workspace,
    whose ticket counters are expected to be zero at every call."""
    import math
    import torch
    import rope_rotation_splice_amd as rrs
    from tests.test_gpu_decode import _setup
    host, devs = _setup(2, 128, [3000, 4000], bt_stride=64, keys=(11,))
    rrs.mla_decode_rotate_on_read(devs["qn"], devs["qr"], devs["cache"], 0, devs["bt"], devs["pend"],
                                  devs["lens"], 1.0 / math.sqrt(576.0), max_seq_len=64 * 64)
    torch.cuda.synchronize()
    assert rrs.device_errors() == 0
    _run(rc.MLA, 2, 4, 16, [(64, 10, 30, 5, 0), (60, 0, 2, 4, 0)], keys=(12,))


def test_debug_checks_refuse_shared_or_bad_written_blocks(monkeypatch):
    """With KVR_DEBUG_CHECKS=1 the splice and the gather refuse, before
    touching memory, a call whose written blocks are shared with another
    logical block (KVR_E_OVERLAP) or lie outside the pool (KVR_E_RANGE); a
    valid call still matches the oracle."""
    import torch
    import rope_rotation_splice_amd as rrs
    monkeypatch.setenv("KVR_DEBUG_CHECKS", "1")
    lay, B, n_blocks = rc.MLA, 16, 12
    pf, rp = rc.random_image(lay, 1, n_blocks * B, (31,))
    cache, keep = rc.to_device(lay, pf, rp, n_blocks, B)
    lens = [60, 60]
    dirs = [(20, 30, 5, 0), (0, 0, 0, 0)]          # sequence 0 writes slots [20, 55): blocks 1..3
    cases = [
        (np.array([[0, 1, 2, 3], [4, 5, 6, 2]], np.int32), -4),    # block 2 also held by sequence 1
        (np.array([[0, 1, 2, 1], [4, 5, 6, 7]], np.int32), -4),    # block 1 held twice by sequence 0
        (np.array([[0, 1, 99, 3], [4, 5, 6, 7]], np.int32), -2),   # outside the pool
    ]
    for bt, code in cases:
        with pytest.raises(rrs.KVRError) as err:
            rrs.leyline_splice(cache, torch.from_numpy(bt).cuda(), lens, dirs)
        assert err.value.status == code
    # the gather: two entries whose destination blocks alias one physical block
    e = torch.zeros((1, 20, 576), dtype=torch.bfloat16, device="cuda")
    ents = [rrs.Rows(e[..., :512], e[..., 512:], 0), rrs.Rows(e[..., :512], e[..., 512:], 0)]
    with pytest.raises(rrs.KVRError) as err:
        rrs.kv_relocate_gather(cache, torch.tensor([0, 1, 2, 1], dtype=torch.int32, device="cuda"), ents, [0, 40])
    assert err.value.status == -4
    torch.cuda.synchronize()
    after = rc.from_device(lay, cache)
    assert np.array_equal(after[0].view(np.uint16), pf.view(np.uint16))
    assert np.array_equal(after[1].view(np.uint16), rp.view(np.uint16))
    assert rrs.device_errors() == 0
    # a valid batch passes the checks and the oracle
    _run(rc.MLA, 2, 16, 16, [(250, 20, 30, 5, 0), (200, 64, 70, 40, 0), (100, 10, 50, 0, 1)], (32,))


def test_ticket_counter_left_nonzero_is_reported_and_recovered():
    """The ticketed mover on a workspace whose ticket counter was left
    nonzero: every workgroup of that (sequence, layer) draws a ticket past
    its tile count, raises KVR_DEV_BAD_TICKET and returns; the launch is
    marked aborted, so no tile stores over sources that may not have been
    read, and every workgroup exits (none waits on a tile that will never
    publish).  device_errors() reports the bit and zeroes the cached splice
    workspaces, after which the same splice on a fresh image matches the
    oracle."""
    import torch
    import rope_rotation_splice_amd as rrs
    from rope_rotation_splice_amd import _abi, api
    lay, B = rc.MLA, 64
    seqs = [(1000, 50, 52, 1, 0), (900, 10, 12, 0, 0)]      # Delta -1 and -2: chains of 64+ bands, ticketed
    lens, dirs = [s[0] for s in seqs], [s[1:] for s in seqs]
    pf, rp = rc.random_image(lay, 2, 2 * 16 * B, (83,))
    cache, keep = rc.to_device(lay, pf, rp, 32, B)
    bt = torch.arange(32, dtype=torch.int32, device="cuda").reshape(2, 16)
    assert rrs.device_errors() == 0
    need = rrs.splice_workspace_bytes(cache, lens, dirs)
    assert need > 0
    ws = api._workspace(need, cache.device, "splice")
    ws.view(torch.int32)[0] = 1 << 20          # counter of (sequence 0, layer 0) past its tile count
    rrs.leyline_splice(cache, bt, lens, dirs)
    torch.cuda.synchronize()
    bits = rrs.device_errors()
    assert bits & _abi.KVR_DEV_BAD_TICKET
    assert not ws.any(), "device_errors() must zero the cached splice workspace"
    assert rrs.device_errors() == 0
    _run(lay, 2, B, 16, [s for s in seqs], (83,), stubs_on=False)
