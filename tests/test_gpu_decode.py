"""Parity of mla_decode_rotate_on_read (HIP, through the C ABI) against the
fp64 oracle: absorbed-MLA decode attention on keys explicitly re-rotated by
each block's pending shift."""

import math

import numpy as np
import pytest

import kvsynth
from oracle import bf16 as ob, decode as odec, rope as orope, splice as osplice, tolerance

pytestmark = pytest.mark.gpu

TH = orope.inv_freq(64, 10000.0)


def _setup(batch, heads, lens, bt_stride, n_layers=1, layer=0, keys=(0,), spare=3, delta_max=100000,
           zero_delta=False):
    import torch
    import rope_rotation_splice_amd as rrs
    r = kvsynth.rng(5, *keys)
    n_blocks = batch * bt_stride + spare
    bt = r.permutation(n_blocks)[: batch * bt_stride].astype(np.int32).reshape(batch, bt_stride)
    pend = r.integers(-delta_max, delta_max, size=(batch, bt_stride), endpoint=True).astype(np.int32)
    if zero_delta:
        pend[:] = 0
    pool = kvsynth.bf16_normal(r, (n_layers, n_blocks * 64, 576))
    qn = kvsynth.bf16_normal(r, (batch, heads, 512))
    qr = kvsynth.bf16_normal(r, (batch, heads, 64))
    dev = lambda a, dt=torch.bfloat16: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(dt).cuda()
    tpool = dev(pool).reshape(n_layers, n_blocks, 64, 576)
    cache = rrs.KVCache.mla(tpool)
    host = dict(bt=bt, pend=pend, pool=pool, qn=qn, qr=qr, lens=np.asarray(lens, np.int32), layer=layer)
    devs = dict(cache=cache, pool=tpool, qn=dev(qn), qr=dev(qr), bt=torch.from_numpy(bt).cuda(),
                pend=torch.from_numpy(pend).cuda(), lens=torch.from_numpy(host["lens"]).cuda())
    return host, devs


def _run(devs, scale, max_len):
    import torch
    import rope_rotation_splice_amd as rrs
    out, lse = rrs.mla_decode_rotate_on_read(devs["qn"], devs["qr"], devs["cache"], 0 if "layer" not in devs else devs["layer"],
                                             devs["bt"], devs["pend"], devs["lens"], scale, max_seq_len=max_len)
    torch.cuda.synchronize()
    assert rrs.device_errors() == 0
    o = out.view(torch.int16).cpu().numpy().view(np.uint16)
    return ob.to_f64(o), lse.cpu().numpy().astype(np.float64)


def _oracle(host, b, scale, pend=None, round_keys=False):
    """(O, LSE, eps_s) of sequence b from the fp64 oracle: keys explicitly
    re-rotated and kept unrounded (or, with round_keys, rounded to bf16 as a
    stored shifted key would be).  eps_s bounds the score change from a key
    one bf16 ulp away; only the planted-needle tests, whose keys are 40x
    larger than the rest, add it to the LSE bar."""
    n = int(host["lens"][b])
    slots = np.arange(n)
    phys = osplice.physical_rows(slots, host["bt"][b], 64)
    rows = host["pool"][host["layer"]][phys]
    ckv = ob.to_f64(rows[:, :512])
    kr = ob.to_f64(rows[:, 512:])
    p = host["pend"] if pend is None else pend
    d = odec.token_deltas(p[b], n, 64)
    qr = ob.to_f64(host["qr"][b])
    o, lse = odec.mla_decode(ob.to_f64(host["qn"][b]), qr, ckv, kr, d, scale, TH, round_keys=round_keys)
    return o, lse, odec.score_bound(qr, kr, d, scale, TH)


@pytest.mark.parametrize("heads", [32, 64, 96, 128])
def test_decode_small(heads):
    lens = [64, 100, 1000, 2048 + 17]
    host, devs = _setup(4, heads, lens, bt_stride=40, keys=(1, heads))
    scale = 1.0 / math.sqrt(576.0)
    o, lse = _run(devs, scale, max_len=40 * 64)
    for b in range(len(lens)):
        o_ref, l_ref, _ = _oracle(host, b, scale)
        ok = tolerance.decode_close(o[b], o_ref, lse[b], l_ref)
        assert ok.all(), f"seq {b}: {(~ok).sum()} heads outside tolerance; worst lse err " \
                         f"{np.abs(lse[b] - l_ref).max():.3g}"


def test_decode_layer_offset_and_many_splits():
    """Layer 2 of 3, sequences long enough for several splits, and a
    one-token sequence.  A single key is not averaged by the softmax: its LSE
    is its score, so the bf16 rounding of its rotated k_r (a matrix-core
    operand) shows in full -- up to scale * 2^-9 * sum |q_r| |k_r|, 3e-3 here
    at scale 0.07.  That sequence is compared with the oracle variant whose
    shifted keys are rounded to bf16; the long ones with the unrounded one."""
    lens = [3000, 1, 2500]
    host, devs = _setup(3, 128, lens, bt_stride=50, n_layers=3, layer=2, keys=(2,))
    devs["layer"] = 2
    scale = 0.07
    o, lse = _run(devs, scale, max_len=50 * 64)
    for b in range(len(lens)):
        o_ref, l_ref, _ = _oracle(host, b, scale, round_keys=lens[b] == 1)
        rel = np.linalg.norm(o[b] - o_ref, axis=1) / np.linalg.norm(o_ref, axis=1)
        assert tolerance.decode_close(o[b], o_ref, lse[b], l_ref).all(), \
            f"seq {b}: max rel-L2 {rel.max():.3g}, max |dLSE| {np.abs(lse[b] - l_ref).max():.3g}"


def test_decode_empty_sequence():
    """A sequence with no cached token attends to nothing: O = 0, LSE = -inf;
    its neighbours in the batch are unaffected."""
    import rope_rotation_splice_amd as rrs
    lens = [0, 70, 0, 64]
    host, devs = _setup(4, 64, lens, bt_stride=4, keys=(4,))
    scale = 1.0 / math.sqrt(576.0)
    o, lse = _run(devs, scale, max_len=4 * 64)
    for b in (0, 2):
        assert (o[b] == 0).all() and np.isneginf(lse[b]).all()
    for b in (1, 3):
        o_ref, l_ref, _ = _oracle(host, b, scale)
        assert tolerance.decode_close(o[b], o_ref, lse[b], l_ref).all()
    assert rrs.device_errors() == 0


def test_decode_large_logits_restart():
    """Scores that jump far above the first tile's maximum (a sharp needle late
    in a split) exercise the restart path: still exact to tolerance."""
    lens = [2048]
    host, devs = _setup(1, 128, lens, bt_stride=32, keys=(3,))
    import torch
    # plant a needle at token 1900 whose correctly rotated k_r is 40 x q_rope
    b, t = 0, 1900
    phys = int(osplice.physical_rows([t], host["bt"][b], 64)[0])
    d = int(host["pend"][b][t // 64])
    qr = ob.to_f64(host["qr"][b][0])
    k = orope.rotate(qr * 40.0, -d, 1, 64, TH)
    host["pool"][0][phys, 512:] = ob.round_rne(k)
    devs["pool"].view(-1, 576)[phys, 512:] = torch.from_numpy(host["pool"][0][phys, 512:].view(np.int16)).view(
        torch.bfloat16).cuda()
    scale = 1.0 / math.sqrt(576.0)
    o, lse = _run(devs, scale, max_len=2048)
    o_ref, l_ref, eps = _oracle(host, b, scale, round_keys=True)
    assert tolerance.decode_close(o[b], o_ref, lse[b], l_ref, eps).all()
    ckv_needle = ob.to_f64(host["pool"][0][phys, :512])
    cos = float(o[b][0] @ ckv_needle / np.linalg.norm(o[b][0]) / np.linalg.norm(ckv_needle))
    assert cos > 0.9


def test_decode_rounded_key_variant_small():
    """Against the oracle variant whose shifted keys are rounded to bf16 (the
    keys an eager relocation would have stored) the device is within the same
    flat bar: the kernel's own bf16 key operands sit between the two."""
    lens = [1000, 2000]
    host, devs = _setup(2, 128, lens, bt_stride=32, keys=(6,))
    scale = 1.0 / math.sqrt(576.0)
    o, lse = _run(devs, scale, max_len=32 * 64)
    for b in range(2):
        n = int(host["lens"][b])
        phys = osplice.physical_rows(np.arange(n), host["bt"][b], 64)
        rows = host["pool"][0][phys]
        d = odec.token_deltas(host["pend"][b], n, 64)
        qr = ob.to_f64(host["qr"][b])
        o_ref, l_ref = odec.mla_decode(ob.to_f64(host["qn"][b]), qr, ob.to_f64(rows[:, :512]),
                                       ob.to_f64(rows[:, 512:]), d, scale, TH, round_keys=True)
        assert tolerance.decode_close(o[b], o_ref, lse[b], l_ref).all()


def test_decode_negative_control_zero_delta():
    """With the pending shifts ignored the output must fail the tolerance
    against the oracle on rotated keys (the rotation is really applied)."""
    lens = [1000, 1500]
    host, devs = _setup(2, 128, lens, bt_stride=24, keys=(4,))
    import torch
    scale = 1.0 / math.sqrt(576.0)
    devs["pend"] = torch.zeros_like(devs["pend"])
    o, lse = _run(devs, scale, max_len=24 * 64)
    for b in range(2):
        o_ref, l_ref, _ = _oracle(host, b, scale)
        assert not tolerance.decode_close(o[b], o_ref, lse[b], l_ref).all()
        o0, l0, _ = _oracle(host, b, scale, pend=np.zeros_like(host["pend"]))
        assert tolerance.decode_close(o[b], o0, lse[b], l0).all()


def test_decode_workload_every_sequence():
    """The full decode workload (batch 32, 32768 tokens, 128 heads, pending
    delta ~ U{-1e5..1e5} per 64-token block) in the launch configuration the
    benchmark times; every sequence is compared with the oracle on
    explicitly re-rotated, unrounded keys at the flat bar (relative L2 2^-8,
    max 2^-7, |dLSE| 2e-3), and sequences 0, 13 and 31 also with the
    rounded-key variant at the same bar.  The measured errors are printed."""
    import torch
    import rope_rotation_splice_amd as rrs
    w = kvsynth.rotate_on_read_decode()
    pool = torch.empty((1, w.n_blocks, 64, 576), dtype=torch.bfloat16, device="cuda")
    kvsynth.fill_normal_(pool, 5, 1)
    qn = torch.empty((w.batch, w.heads, 512), dtype=torch.bfloat16, device="cuda")
    qr = torch.empty((w.batch, w.heads, 64), dtype=torch.bfloat16, device="cuda")
    kvsynth.fill_normal_(qn, 5, 2)
    kvsynth.fill_normal_(qr, 5, 3)
    cache = rrs.KVCache.mla(pool)
    bt = torch.from_numpy(w.block_tables).cuda()
    pend = torch.from_numpy(w.pending_delta).cuda()
    lens = torch.from_numpy(w.seq_lens).cuda()
    out, lse = rrs.mla_decode_rotate_on_read(qn, qr, cache, 0, bt, pend, lens, w.scale, max_seq_len=w.ctx)
    torch.cuda.synchronize()
    assert rrs.device_errors() == 0
    o = ob.to_f64(out.view(torch.int16).cpu().numpy().view(np.uint16))
    lse = lse.cpu().numpy().astype(np.float64)
    h16 = lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)
    qn_h, qr_h = h16(qn), h16(qr)
    for b in range(w.batch):
        phys = osplice.physical_rows(np.arange(w.ctx), w.block_tables[b], 64)
        rows = h16(pool[0].reshape(-1, 576)[torch.from_numpy(phys).cuda()])
        d = odec.token_deltas(w.pending_delta[b], w.ctx, 64)
        kr = ob.to_f64(rows[:, 512:])
        for rk in ((False, True) if b in (0, 13, 31) else (False,)):
            o_ref, l_ref = odec.mla_decode(ob.to_f64(qn_h[b]), ob.to_f64(qr_h[b]), ob.to_f64(rows[:, :512]),
                                           kr, d, w.scale, TH, round_keys=rk)
            rel = np.linalg.norm(o[b] - o_ref, axis=1) / np.linalg.norm(o_ref, axis=1)
            dl = np.abs(lse[b] - l_ref)
            print(f"seq {b} keys {'rounded' if rk else 'unrounded'}: max rel-L2 {rel.max():.3e}, "
                  f"max |dLSE| {dl.max():.3e}, mean |dLSE| {dl.mean():.3e}")
            ok = tolerance.decode_close(o[b], o_ref, lse[b], l_ref)
            assert ok.all(), f"seq {b} ({'rounded' if rk else 'unrounded'} keys): {(~ok).sum()} heads outside"


def test_decode_nan_rows_past_length():
    """Cache rows past a sequence's length (same block, and whole blocks the
    table still names) may hold anything, NaN included: masked tokens get
    P = 0 and must not contribute 0 * NaN to O."""
    import torch
    lens = [100, 64 * 3 + 5, 1]
    host, devs = _setup(3, 128, lens, bt_stride=8, keys=(7,))
    nan = np.uint16(0x7FC0)
    for b, n in enumerate(lens):
        for t in range(n, 8 * 64):
            phys = int(osplice.physical_rows([t], host["bt"][b], 64)[0])
            devs["pool"].view(-1, 576)[phys] = torch.from_numpy(
                np.full(576, nan, np.uint16).view(np.int16)).view(torch.bfloat16).cuda()
    scale = 1.0 / math.sqrt(576.0)
    o, lse = _run(devs, scale, max_len=8 * 64)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    for b in range(len(lens)):
        # a one-token sequence is checked against rounded keys (see the layer-offset test)
        o_ref, l_ref, _ = _oracle(host, b, scale, round_keys=lens[b] == 1)
        assert tolerance.decode_close(o[b], o_ref, lse[b], l_ref).all(), f"seq {b}"
