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


def test_gqa_gather_patch_block_size_not_a_power_of_two():
    # 24-row blocks take the register-tiled kernel, which divides slots by the block size
    chunks = [(96, 30000, 5, None), (17, 0, 200, None), (130, 9000, 230, None)]
    _run(rc.GQA, 2, 24, 16, 2, chunks, 16, 1.0, (25,))


def test_gqa_gather_patch_long_entries():
    # entries of more than 64 sixteen-row stages span several row chunks of
    # the streaming kernel (1500 rows: 94 stages, the last one ragged)
    chunks = [(1500, 1234, 64, None), (1025, 0, 2000, None), (16, 70000, 3100, None)]
    _run(rc.GQA, 2, 64, 52, 2, chunks, 16, 1.0, (26,))


def test_gather_patch_keys_only_and_zero_shift():
    chunks = [(40, 40, 40, None), (70, 1000, 100, None)]     # first entry: delta = 0
    _run(rc.GQA, 2, 64, 4, 1, chunks, 16, 1.0, (23,), patch_pf=False)


def test_mla_gather_patch_both_channels():
    """Kamera patches both MLA channels: cKV (512) and k_rope (64)."""
    chunks = [(100, 60000, 3, None), (64, 0, 200, None), (1, 7, 300, None)]
    _run(rc.MLA, 3, 64, 6, 2, chunks, 16, 1.0, (24,))


@pytest.mark.parametrize("part,ranges", [(0, [(5, 96), (200, 64), (300, 17), (400, 0)]),
                                         (1, [(5, 96), (200, 64), (300, 17), (400, 0)]),
                                         (0, [(3, 1100), (1200, 33)]), (1, [(40, 1041)])])
def test_patch_in_place(part, ranges):
    import torch
    import rope_rotation_splice_amd as rrs
    lay = rc.GQA
    L, B, n_dst, spare = 2, 16, 80, 3
    r = kvsynth.rng(25, part, len(ranges))
    n_blocks = n_dst + spare
    bt = r.permutation(n_blocks)[:n_dst].astype(np.int32)
    pf, rp = rc.random_image(lay, L, n_blocks * B, (25, part))
    cache, keep = rc.to_device(lay, pf, rp, n_blocks, B)
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


def test_gqa_patch_workload_every_layer():
    """The full GQA workload (32 layers, 16 chunks x 1024 tokens, rank 16,
    factors N(0, 0.01^2)) in the launch configuration the benchmark times;
    every layer of every chunk is compared in full with the oracle."""
    import torch
    import rope_rotation_splice_amd as rrs
    w = kvsynth.gqa_patch()
    lay = rc.GQA
    L, B, width, m = w.shape.n_layers, w.block_size, w.shape.width, w.rank
    K = torch.empty((L, w.n_blocks, B, width), dtype=torch.bfloat16, device="cuda")
    V = torch.empty_like(K)
    kvsynth.fill_normal_(K, 4, 1)
    kvsynth.fill_normal_(V, 4, 2)
    cache = rrs.KVCache.gqa(K, V, 8, 128, 500000.0)
    ents, fk, fv, keep = [], [], [], []
    for i in range(len(w.deltas)):
        ek = torch.empty((L, w.chunk_len, width), dtype=torch.bfloat16, device="cuda")
        ev = torch.empty_like(ek)
        kvsynth.fill_normal_(ek, 4, 3, i, 0)
        kvsynth.fill_normal_(ev, 4, 3, i, 1)
        fac = []
        for j in range(4):
            t = torch.empty((L, w.chunk_len if j % 2 == 0 else width, m), dtype=torch.float32, device="cuda")
            kvsynth.fill_normal_(t, 4, 4, i, j, std=w.factor_std)
            fac.append(t)
        ents.append(rrs.Rows(ev, ek, int(w.base_pos[i])))
        fk.append(rrs.LowRank(fac[0], fac[1]))
        fv.append(rrs.LowRank(fac[2], fac[3]))
        keep.append((ek, ev, fac))
    layers = range(L)
    h16 = lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)
    before_k = {l: h16(K[l]).reshape(-1, width) for l in layers}
    before_v = {l: h16(V[l]).reshape(-1, width) for l in layers}
    rrs.kv_relocate_gather(cache, torch.from_numpy(w.block_table).cuda(), ents, w.p_target.tolist(), fk, fv)
    torch.cuda.synchronize()
    assert rrs.device_errors() == 0
    for l in layers:
        ak = h16(K[l]).reshape(-1, width)
        av = h16(V[l]).reshape(-1, width)
        entries = [(h16(ev[l])[None], h16(ek[l])[None], int(w.base_pos[i])) for i, (ek, ev, _) in enumerate(keep)]
        fr = [(f[0][l:l + 1].cpu().numpy(), f[1][l:l + 1].cpu().numpy()) for (_, _, f) in keep]
        fp = [(f[2][l:l + 1].cpu().numpy(), f[3][l:l + 1].cpu().numpy()) for (_, _, f) in keep]
        rc.check_gather_patch(lay, (before_v[l][None], before_k[l][None]), (av[None], ak[None]), w.block_table, B,
                              entries, w.p_target.tolist(), fr, fp)
