"""Parity of kv_relocate_gather (HIP, through the C ABI) against the fp64 oracle."""

import numpy as np
import pytest

import kvsynth
from tests import relocation_cases as rc

pytestmark = pytest.mark.gpu


def _run(lay, n_layers, block_size, n_dst_blocks, spare, chunks, keys):
    """chunks: list of (len, base_pos, p_target)."""
    import torch
    import rope_rotation_splice_amd as rrs
    n_blocks = n_dst_blocks + spare
    r = kvsynth.rng(*keys, 7)
    bt = r.permutation(n_blocks)[:n_dst_blocks].astype(np.int32)
    pf, rp = rc.random_image(lay, n_layers, n_blocks * block_size, keys)
    cache, keep = rc.to_device(lay, pf, rp, n_blocks, block_size)
    d_bt = torch.from_numpy(bt).cuda()
    ents_h, ents_d = [], []
    for i, (ln, base, pt) in enumerate(chunks):
        epf, erp = rc.random_image(lay, n_layers, ln, keys + (300 + i,))
        ents_h.append((epf, erp, base))
        tp, tr = rc.rows_to_device(lay, epf, erp)
        ents_d.append(rrs.Rows(tp, tr, base))
    rrs.kv_relocate_gather(cache, d_bt, ents_d, [c[2] for c in chunks])
    torch.cuda.synchronize()
    after = rc.from_device(lay, cache)
    assert rrs.device_errors() == 0
    rc.check_gather(lay, (pf, rp), after, bt, block_size, ents_h, [c[2] for c in chunks])


@pytest.mark.parametrize("block_size", [1, 4, 64])
def test_gather_small_mla(block_size):
    n_dst = 2048 // block_size
    chunks = [(300, 60000, 5), (1, 0, 400), (0, 5, 500), (129, 700, 700), (1000, 31, 1040)]
    _run(rc.MLA, 3, block_size, n_dst, 5, chunks, (block_size, 11))


def test_gather_block_size_not_a_power_of_two():
    # 24-row blocks: the kernel divides slots by the block size instead of shifting
    chunks = [(300, 60000, 5), (1, 0, 400), (129, 700, 700), (250, 31, 1000)]
    _run(rc.MLA, 3, 24, 1280 // 24, 5, chunks, (24, 11))


def test_gather_many_entries_multiple_launches():
    r = kvsynth.rng(12)
    chunks, pos = [], 3
    for i in range(40):
        ln = int(r.integers(1, 70))
        chunks.append((ln, int(r.integers(0, 100000)), pos))
        pos += ln + int(r.integers(0, 5))
    _run(rc.MLA, 2, 16, (pos + 15) // 16, 4, chunks, (13,))


def test_gather_gqa_and_fp32():
    chunks = [(200, 30000, 64), (77, 0, 300), (333, 9000, 400)]
    _run(rc.GQA, 2, 64, 12, 2, chunks, (14,))
    _run(rc.MLA_F32, 2, 32, 24, 2, chunks, (15,))


def test_gather_registry_workload_every_layer():
    """The 61-layer registry workload at full size (32 entries into a
    40960-slot paged sequence), in the launch configuration the benchmark
    times: every layer is compared in full with the oracle (moved rows,
    untouched rows and canaries), then a random sample of rows is recomputed
    one by one."""
    import torch
    import rope_rotation_splice_amd as rrs
    w = kvsynth.registry_gather()
    lay = rc.MLA
    L, B = w.shape.n_layers, w.block_size
    rows = w.n_blocks * B
    pool = torch.empty((L, w.n_blocks, B, 576), dtype=torch.bfloat16, device="cuda")
    kvsynth.fill_normal_(pool, 2, 1)
    cache = rrs.KVCache.mla(pool)
    ents, ents_d = [], []
    for i in range(len(w.lens)):
        ln = int(w.lens[i])
        e = torch.empty((L, ln, 576), dtype=torch.bfloat16, device="cuda")
        kvsynth.fill_normal_(e, 2, 2, i)
        ents.append(e)
        ents_d.append(rrs.Rows(e[..., :512], e[..., 512:], int(w.base_pos[i])))
    d_bt = torch.from_numpy(w.block_table).cuda()
    before = pool.view(torch.int16).cpu().numpy().view(np.uint16).reshape(L, rows, 576)
    rrs.kv_relocate_gather(cache, d_bt, ents_d, w.p_target.tolist())
    torch.cuda.synchronize()
    assert rrs.device_errors() == 0
    after = pool.view(torch.int16).cpu().numpy().view(np.uint16).reshape(L, rows, 576)
    ent_h = [e.view(torch.int16).cpu().numpy().view(np.uint16) for e in ents]
    for l in range(L):
        rc.check_gather(lay, (before[l:l + 1, :, :512], before[l:l + 1, :, 512:]),
                        (after[l:l + 1, :, :512], after[l:l + 1, :, 512:]), w.block_table, B,
                        [(e[l:l + 1, :, :512], e[l:l + 1, :, 512:], int(w.base_pos[i])) for i, e in enumerate(ent_h)],
                        w.p_target.tolist())
    # sampled rows of every layer
    from oracle import gather as og, splice as osp, tolerance
    th = lay.theta()
    r = kvsynth.rng(2, 3)
    for _ in range(2000):
        l = int(r.integers(0, L))
        c = int(r.integers(0, len(w.lens)))
        t = int(r.integers(0, int(w.lens[c])))
        phys = int(osp.physical_rows([int(w.p_target[c]) + t], w.block_table, B)[0])
        d = og.chunk_delta(int(w.p_target[c]), int(w.base_pos[c]))
        src = ent_h[c][l, t]
        opf, ref, norm, _ = og.relocate_rows(src[None, :512], src[None, 512:], d, 1, 64, th)
        assert np.array_equal(after[l, phys, :512], opf[0])
        assert tolerance.bf16_close(after[l, phys, 512:], ref[0], norm[0]).all()
