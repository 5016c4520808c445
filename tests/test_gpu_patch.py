"""Parity of the rank-m patch path (fused into the gather, and in place)
against the fp64 oracle: K_out = R(delta) K + U V^T, V_out = V + U' V'^T."""

import numpy as np
import pytest

import kvsynth
from oracle import bf16 as ob, patch as opatch, splice as osplice, tolerance
from tests import relocation_cases as rc

pytestmark = pytest.mark.gpu


def _factors(L, n, width, rank, std, keys):
    r = kvsynth.rng(*keys)
    return kvsynth.f32_normal(r, (L, n, rank), std), kvsynth.f32_normal(r, (L, width, rank), std)


def _dev(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _run(lay, n_layers, block_size, n_dst, spare, chunks, rank, std, keys, patch_rope=True, patch_pf=True):
    """chunks: list of (len, base_pos, p_target, rank or None)."""
    import torch
    import rope_rotation_splice_amd as rrs
    n_blocks = n_dst + spare
    r = kvsynth.rng(*keys, 7)
    bt = r.permutation(n_blocks)[:n_dst].astype(np.int32)
    pf, rp = rc.random_image(lay, n_layers, n_blocks * block_size, keys)
    cache, keep = rc.to_device(lay, pf, rp, n_blocks, block_size)
    d_bt = torch.from_numpy(bt).cuda()
    ents_h, ents_d, fr_h, fp_h, fr_d, fp_d = [], [], [], [], [], []
    for i, (ln, base, pt, rk) in enumerate(chunks):
        epf, erp = rc.random_image(lay, n_layers, ln, keys + (300 + i,))
        ents_h.append((epf, erp, base))
        tp, tr = rc.rows_to_device(lay, epf, erp)
        ents_d.append(rrs.Rows(tp, tr, base))
        rk = rank if rk is None else rk
        for on, width, hl, dl, k2 in ((patch_rope, lay.rope_width, fr_h, fr_d, 1), (patch_pf, lay.pf_width, fp_h, fp_d, 2)):
            if on and rk > 0:
                U, V = _factors(n_layers, ln, width, rk, std, keys + (600 + i, k2))
                hl.append((U, V))
                dl.append(rrs.LowRank(_dev(U), _dev(V)))
            else:
                hl.append(None)
                dl.append(None)
    rrs.kv_relocate_gather(cache, d_bt, ents_d, [c[2] for c in chunks], fr_d, fp_d)
    torch.cuda.synchronize()
    after = rc.from_device(lay, cache)
    assert rrs.device_errors() == 0
    rc.check_gather_patch(lay, (pf, rp), after, bt, block_size, ents_h, [c[2] for c in chunks], fr_h, fp_h)


@pytest.mark.parametrize("std", [1.0, 0.01])
def test_gqa_gather_patch_rank16(std):
    # 96 tokens x 1024 features: tokens != features, so a transposed patch fails
    chunks = [(96, 30000, 64, None), (17, 0, 200, None), (64, 9000, 256, None), (130, 5, 400, None)]
    _run(rc.GQA, 2, 64, 10, 2, chunks, 16, std, (21, int(std * 100)))


@pytest.mark.parametrize("rank", [4, 12, 32, 64])
def test_gqa_gather_patch_ranks(rank):
    chunks = [(50, 1000, 10, None), (77, 99999, 100, 0), (33, 0, 190, None)]
    _run(rc.GQA, 2, 16, 16, 2, chunks, rank, 1.0, (22, rank))


def test_gather_patch_keys_only_and_zero_shift():
    chunks = [(40, 40, 40, None), (70, 1000, 100, None)]     # first entry: delta = 0
    _run(rc.GQA, 2, 64, 4, 1, chunks, 16, 1.0, (23,), patch_pf=False)


def test_mla_gather_patch_both_channels():
    """Kamera patches both MLA channels: cKV (512) and k_rope (64)."""
    chunks = [(100, 60000, 3, None), (64, 0, 200, None), (1, 7, 300, None)]
    _run(rc.MLA, 3, 64, 6, 2, chunks, 16, 1.0, (24,))


@pytest.mark.parametrize("part", [0, 1])
def test_patch_in_place(part):
    import torch
    import rope_rotation_splice_amd as rrs
    lay = rc.GQA
    L, B, n_dst, spare = 2, 16, 40, 3
    r = kvsynth.rng(25, part)
    n_blocks = n_dst + spare
    bt = r.permutation(n_blocks)[:n_dst].astype(np.int32)
    pf, rp = rc.random_image(lay, L, n_blocks * B, (25, part))
    cache, keep = rc.to_device(lay, pf, rp, n_blocks, B)
    ranges = [(5, 96), (200, 64), (300, 17), (400, 0)]
    width = lay.pf_width if part == 0 else lay.rope_width
    fh, fd = [], []
    for i, (p, n) in enumerate(ranges):
        U, V = _factors(L, n, width, 16, 1.0, (25, part, i))
        fh.append((U, V))
        fd.append(rrs.LowRank(_dev(U), _dev(V)))
    rrs.kv_patch_lowrank(cache, torch.from_numpy(bt).cuda(), part, [p for p, _ in ranges], [n for _, n in ranges], fd)
    torch.cuda.synchronize()
    pf1, rp1 = rc.from_device(lay, cache)
    assert rrs.device_errors() == 0
    before, after = (pf, pf1) if part == 0 else (rp, rp1)
    other0, other1 = (rp, rp1) if part == 0 else (pf, pf1)
    assert np.array_equal(other0, other1)
    touched = np.zeros(before.shape[1], bool)
    for (p, n), (U, V) in zip(ranges, fh):
        if n == 0:
            continue
        phys = osplice.physical_rows(p + np.arange(n), bt, B)
        touched[phys] = True
        for l in range(L):
            x = ob.to_f64(before[l][phys])
            y = opatch.patch_values(x, U[l], V[l])
            ok = tolerance.bf16_close(after[l][phys], y, np.abs(x) + opatch.patch_abs_scale(U[l], V[l]))
            assert ok.all(), f"range {p} layer {l}: {(~ok).sum()} outside tolerance"
    assert np.array_equal(after[:, ~touched], before[:, ~touched])
