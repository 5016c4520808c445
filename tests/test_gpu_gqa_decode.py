"""Parity of gqa_decode_rotate_on_read (HIP, through the C ABI) against the
fp64 oracle: GQA decode attention on keys rotated by each block's pending
shift, query head h reading KV head h // (q_heads / kv_heads)."""

import math

import numpy as np
import pytest

import kvsynth
from oracle import bf16 as ob, decode as odec, rope as orope, splice as osplice, tolerance

pytestmark = pytest.mark.gpu

D = 128
TH = orope.inv_freq(D, 500000.0)


def _setup(batch, q_heads, kv_heads, lens, bt_stride, n_layers=1, layer=0, keys=(0,), spare=3, delta_max=30000):
    import torch
    import rope_rotation_splice_amd as rrs
    r = kvsynth.rng(7, *keys)
    n_blocks = batch * bt_stride + spare
    bt = r.permutation(n_blocks)[: batch * bt_stride].astype(np.int32).reshape(batch, bt_stride)
    pend = r.integers(-delta_max, delta_max, size=(batch, bt_stride), endpoint=True).astype(np.int32)
    W = kv_heads * D
    kpool = kvsynth.bf16_normal(r, (n_layers, n_blocks * 64, W))
    vpool = kvsynth.bf16_normal(r, (n_layers, n_blocks * 64, W))
    q = kvsynth.bf16_normal(r, (batch, q_heads, D))
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    tk = dev(kpool).reshape(n_layers, n_blocks, 64, W)
    tv = dev(vpool).reshape(n_layers, n_blocks, 64, W)
    cache = rrs.KVCache.gqa(tk, tv, kv_heads, D)
    host = dict(bt=bt, pend=pend, k=kpool, v=vpool, q=q, lens=np.asarray(lens, np.int32), layer=layer,
                kv_heads=kv_heads)
    devs = dict(cache=cache, k=tk, v=tv, q=dev(q), bt=torch.from_numpy(bt).cuda(),
                pend=torch.from_numpy(pend).cuda(), lens=torch.from_numpy(host["lens"]).cuda(), layer=layer)
    return host, devs


def _run(devs, scale, max_len, expect_errors=0):
    import torch
    import rope_rotation_splice_amd as rrs
    out, lse = rrs.gqa_decode_rotate_on_read(devs["q"], devs["cache"], devs["layer"], devs["bt"], devs["pend"],
                                             devs["lens"], scale, max_seq_len=max_len)
    torch.cuda.synchronize()
    assert rrs.device_errors() == expect_errors
    o = out.view(torch.int16).cpu().numpy().view(np.uint16)
    return ob.to_f64(o), lse.cpu().numpy().astype(np.float64)


def _oracle(host, b, scale, pend=None, skip_blocks=()):
    """(O, LSE, eps_s) of sequence b from the fp64 oracle."""
    n = int(host["lens"][b])
    slots = np.array([t for t in range(n) if t // 64 not in skip_blocks], np.int64)
    phys = osplice.physical_rows(slots, host["bt"][b], 64)
    k = ob.to_f64(host["k"][host["layer"]][phys])
    v = ob.to_f64(host["v"][host["layer"]][phys])
    p = host["pend"] if pend is None else pend
    d = odec.token_deltas(p[b], n, 64)[slots] if n else np.zeros(0, np.int64)
    q = ob.to_f64(host["q"][b])
    o, lse = odec.gqa_decode(q, k, v, d, scale, TH, host["kv_heads"])
    return o, lse, odec.gqa_score_bound(q, k, d, scale, TH, host["kv_heads"])


def _check(o, lse, host, scale, seqs, **kw):
    for b in seqs:
        o_ref, l_ref, _ = _oracle(host, b, scale, **kw)
        ok = tolerance.decode_close(o[b], o_ref, lse[b], l_ref)
        rel = np.linalg.norm(o[b] - o_ref, axis=1) / np.linalg.norm(o_ref, axis=1)
        assert ok.all(), f"seq {b}: {(~ok).sum()} heads outside tolerance; max rel-L2 {rel.max():.3g}, " \
                         f"max |dLSE| {np.abs(lse[b] - l_ref).max():.3g}"


@pytest.mark.parametrize("q_heads,kv_heads", [(32, 8), (8, 8), (16, 8), (32, 2), (64, 4), (64, 8), (24, 8),
                                                (40, 8), (21, 3)])
def test_gqa_decode_small(q_heads, kv_heads):
    lens = [64, 100, 1000, 2048 + 17, 1, 33]
    host, devs = _setup(len(lens), q_heads, kv_heads, lens, bt_stride=40, keys=(1, q_heads, kv_heads))
    scale = 1.0 / math.sqrt(D)
    o, lse = _run(devs, scale, max_len=40 * 64)
    _check(o, lse, host, scale, range(len(lens)))


def test_gqa_decode_layer_offset_and_many_splits():
    """Layer 2 of 3, and sequences long enough to need several splits of at
    most 64 blocks each."""
    lens = [3000, 1, 6400, 4097]
    host, devs = _setup(4, 32, 8, lens, bt_stride=100, n_layers=3, layer=2, keys=(2,))
    scale = 0.07
    o, lse = _run(devs, scale, max_len=100 * 64)
    _check(o, lse, host, scale, range(len(lens)))


def test_gqa_decode_empty_sequence():
    import rope_rotation_splice_amd as rrs
    lens = [0, 70]
    host, devs = _setup(2, 32, 8, lens, bt_stride=4, keys=(3,))
    scale = 1.0 / math.sqrt(D)
    o, lse = _run(devs, scale, max_len=4 * 64)
    assert (o[0] == 0).all() and np.isneginf(lse[0]).all()
    _check(o, lse, host, scale, [1])
    assert rrs.device_errors() == 0


def test_gqa_decode_negative_control_zero_delta():
    """With the pending shifts zeroed on the device the output must fail the
    tolerance against the oracle on the true shifts (the rotation is really
    applied), and match the oracle on zero shifts."""
    import torch
    lens = [1000, 1500]
    host, devs = _setup(2, 32, 8, lens, bt_stride=24, keys=(4,))
    scale = 1.0 / math.sqrt(D)
    devs["pend"] = torch.zeros_like(devs["pend"])
    o, lse = _run(devs, scale, max_len=24 * 64)
    for b in range(2):
        o_ref, l_ref, _ = _oracle(host, b, scale)
        assert not tolerance.decode_close(o[b], o_ref, lse[b], l_ref).all()
    _check(o, lse, host, scale, range(2), pend=np.zeros_like(host["pend"]))


def test_gqa_decode_needle():
    """A key planted at token 1900 so that its correctly rotated form is 6 q
    (query head 0) is retrieved: head 0's output is that token's V row."""
    import torch
    lens = [2048]
    host, devs = _setup(1, 32, 8, lens, bt_stride=32, keys=(5,))
    b, t = 0, 1900
    phys = int(osplice.physical_rows([t], host["bt"][b], 64)[0])
    d = int(host["pend"][b][t // 64])
    q0 = ob.to_f64(host["q"][b][0])
    k = orope.rotate(q0 * 6.0, -d, 1, D, TH)
    host["k"][0][phys, :D] = ob.round_rne(k)
    devs["k"].view(-1, 8 * D)[phys, :D] = torch.from_numpy(host["k"][0][phys, :D].view(np.int16)).view(
        torch.bfloat16).cuda()
    scale = 1.0 / math.sqrt(D)
    o, lse = _run(devs, scale, max_len=2048)
    _check(o, lse, host, scale, [0])
    v_needle = ob.to_f64(host["v"][0][phys, :D])
    cos = float(o[b][0] @ v_needle / np.linalg.norm(o[b][0]) / np.linalg.norm(v_needle))
    assert cos > 0.9


def test_gqa_decode_nan_rows_past_length():
    """Cache rows past a sequence's length (same block, and whole blocks the
    table still names) may hold anything, NaN included."""
    import torch
    lens = [100, 64 * 3 + 5, 1]
    host, devs = _setup(3, 32, 8, lens, bt_stride=8, keys=(6,))
    nan = np.uint16(0x7FC0)
    row = torch.from_numpy(np.full(8 * D, nan, np.uint16).view(np.int16)).view(torch.bfloat16).cuda()
    for b, n in enumerate(lens):
        for t in range(n, 8 * 64):
            phys = int(osplice.physical_rows([t], host["bt"][b], 64)[0])
            devs["k"].view(-1, 8 * D)[phys] = row
            devs["v"].view(-1, 8 * D)[phys] = row
    scale = 1.0 / math.sqrt(D)
    o, lse = _run(devs, scale, max_len=8 * 64)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    _check(o, lse, host, scale, range(len(lens)))


def test_gqa_decode_bad_block_skipped_and_flagged():
    """A block-table entry outside the pool raises KVR_DEV_BAD_BLOCK and its
    tokens take no part; the other tokens are attended as usual."""
    import torch
    lens = [500, 300]
    host, devs = _setup(2, 32, 8, lens, bt_stride=8, keys=(7,))
    bt = devs["bt"].clone()
    bt[0, 2] = 10 ** 6
    devs["bt"] = bt
    scale = 1.0 / math.sqrt(D)
    o, lse = _run(devs, scale, max_len=8 * 64, expect_errors=1)
    _check(o, lse, host, scale, [0], skip_blocks=(2,))
    _check(o, lse, host, scale, [1])


def test_gqa_decode_workload_every_sequence():
    """The full GQA decode workload (batch 32, 32768 tokens, 32 query heads on
    8 KV heads of 128, pending delta ~ U{-30000..30000} per 64-token block) in
    the launch configuration the benchmark times; every sequence is compared
    with the oracle."""
    import torch
    import rope_rotation_splice_amd as rrs
    w = kvsynth.gqa_rotate_on_read_decode()
    G, W = w.shape.heads, w.shape.heads * D
    kp = torch.empty((1, w.n_blocks, 64, W), dtype=torch.bfloat16, device="cuda")
    vp = torch.empty_like(kp)
    q = torch.empty((w.batch, w.q_heads, D), dtype=torch.bfloat16, device="cuda")
    kvsynth.fill_normal_(kp, 7, 1)
    kvsynth.fill_normal_(vp, 7, 2)
    kvsynth.fill_normal_(q, 7, 3)
    cache = rrs.KVCache.gqa(kp, vp, G, D)
    bt = torch.from_numpy(w.block_tables).cuda()
    pend = torch.from_numpy(w.pending_delta).cuda()
    lens = torch.from_numpy(w.seq_lens).cuda()
    out, lse = rrs.gqa_decode_rotate_on_read(q, cache, 0, bt, pend, lens, w.scale, max_seq_len=w.ctx)
    torch.cuda.synchronize()
    assert rrs.device_errors() == 0
    o = ob.to_f64(out.view(torch.int16).cpu().numpy().view(np.uint16))
    lse = lse.cpu().numpy().astype(np.float64)
    h16 = lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)
    q_h = h16(q)
    for b in range(w.batch):
        phys = torch.from_numpy(osplice.physical_rows(np.arange(w.ctx), w.block_tables[b], 64)).cuda()
        k = ob.to_f64(h16(kp[0].reshape(-1, W)[phys]))
        v = ob.to_f64(h16(vp[0].reshape(-1, W)[phys]))
        d = odec.token_deltas(w.pending_delta[b], w.ctx, 64)
        qb = ob.to_f64(q_h[b])
        o_ref, l_ref = odec.gqa_decode(qb, k, v, d, w.scale, TH, G)
        ok = tolerance.decode_close(o[b], o_ref, lse[b], l_ref)
        rel = np.linalg.norm(o[b] - o_ref, axis=1) / np.linalg.norm(o_ref, axis=1)
        print(f"seq {b}: max rel-L2 {rel.max():.3e}, max |dLSE| {np.abs(lse[b] - l_ref).max():.3e}")
        assert ok.all(), f"seq {b}: {(~ok).sum()} heads outside tolerance; max rel-L2 {rel.max():.3g}"
