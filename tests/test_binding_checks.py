"""The Python binding refuses tensors the kernels would misread -- host
tensors, wrong dtypes, short tables, rows or factors that do not match the
cache -- with ValueError, before any library call (so these run without a
GPU: every tensor here is a host tensor, and a check that were missing would
reach the library instead)."""

import pytest
import torch

import rope_rotation_splice_amd as rrs

BF, F32, I32 = torch.bfloat16, torch.float32, torch.int32


def mla(layers=2, blocks=4, rows=16):
    return rrs.KVCache.mla(torch.zeros((layers, blocks, rows, 576), dtype=BF))


def gqa(layers=2, blocks=4, rows=16):
    k = torch.zeros((layers, blocks, rows, 1024), dtype=BF)
    return rrs.KVCache.gqa(k, torch.zeros_like(k), 8, 128)


def rows(layers, n, pf=512, rp=64, dtype=BF):
    return rrs.Rows(torch.zeros((layers, n, pf), dtype=dtype), torch.zeros((layers, n, rp), dtype=dtype))


def test_cache_parts_checked():
    with pytest.raises(ValueError, match="bfloat16 or float32"):
        rrs.KVCache.mla(torch.zeros((1, 1, 4, 576), dtype=torch.float16))


def test_splice_checks():
    c = mla()
    bt = torch.zeros((1, 4), dtype=I32)
    with pytest.raises(ValueError, match="CUDA"):
        rrs.leyline_splice(c, bt, [10], [(1, 2, 1, 0)])
    with pytest.raises(ValueError, match="int32"):
        rrs.leyline_splice(c, bt.long(), [10], [(1, 2, 1, 0)])
    with pytest.raises(ValueError, match="row per directive"):
        rrs.leyline_splice(c, bt, [10, 10], [(1, 2, 1, 0), (1, 2, 1, 0)])
    with pytest.raises(ValueError, match="one length per directive"):
        rrs.leyline_splice(c, bt, [10, 10], [(1, 2, 1, 0)])
    with pytest.raises(ValueError, match="one entry"):
        rrs.leyline_splice(c, bt, [10], [(1, 2, 1, 0)], stubs=[None, None])
    for bad, msg in ((rows(3, 1), "layers"), (rows(2, 1, pf=256), "widths"), (rows(2, 1, dtype=F32), "dtypes")):
        with pytest.raises(ValueError, match=msg):
            rrs.leyline_splice(c, bt, [10], [(1, 2, 1, 0)], stubs=[bad])


def test_lazy_checks():
    bt = torch.zeros((2, 8), dtype=I32)
    with pytest.raises(ValueError, match="CUDA"):
        rrs.leyline_splice_lazy(bt, torch.zeros_like(bt), 64, [128], [(0, 64, 0, 0)])
    with pytest.raises(ValueError, match="row per directive"):
        rrs.leyline_splice_lazy(bt, torch.zeros_like(bt), 64, [128] * 3, [(0, 64, 0, 0)] * 3)
    e = rrs.LazyEntry(5, torch.zeros(2, dtype=I32), 128, 0, 0)
    with pytest.raises(ValueError, match="CUDA"):
        rrs.kv_relocate_gather_lazy(bt, torch.zeros_like(bt), 64, [e])
    with pytest.raises(ValueError, match="match block_tables"):
        rrs.kv_relocate_gather_lazy(bt, torch.zeros((2, 7), dtype=I32), 64, [e])


def test_gather_checks():
    c = mla()
    bt = torch.zeros(4, dtype=I32)
    e = rows(2, 10)
    with pytest.raises(ValueError, match="CUDA"):
        rrs.kv_relocate_gather(c, bt, [e], [0])
    with pytest.raises(ValueError, match="one target per entry"):
        rrs.kv_relocate_gather(c, bt, [e], [0, 5])
    with pytest.raises(ValueError, match="layers"):
        rrs.kv_relocate_gather(c, bt, [rows(1, 10)], [0])
    good = rrs.LowRank(torch.zeros((2, 10, 16)), torch.zeros((2, 64, 16)))
    transposed = rrs.LowRank(torch.zeros((2, 64, 16)), torch.zeros((2, 10, 16)))
    with pytest.raises(ValueError, match="patch_rope\\[0\\].U"):
        rrs.kv_relocate_gather(c, bt, [e], [0], patch_rope=[transposed])
    with pytest.raises(ValueError, match="one entry"):
        rrs.kv_relocate_gather(c, bt, [e], [0], patch_rope=[good, good])
    with pytest.raises(ValueError, match="float32"):
        rrs.kv_relocate_gather(c, bt, [e], [0], patch_pf=[rrs.LowRank(torch.zeros((2, 10, 16), dtype=BF),
                                                                      torch.zeros((2, 512, 16)))])


def test_patch_checks():
    c = gqa()
    bt = torch.zeros(4, dtype=I32)
    f = rrs.LowRank(torch.zeros((2, 8, 16)), torch.zeros((2, 1024, 16)))
    with pytest.raises(ValueError, match="CUDA"):
        rrs.kv_patch_lowrank(c, bt, 1, [0], [8], [f])
    with pytest.raises(ValueError, match="part must be"):
        rrs.kv_patch_lowrank(c, bt, 2, [0], [8], [f])
    with pytest.raises(ValueError, match="shape"):
        rrs.kv_patch_lowrank(c, bt, 1, [0], [9], [f])
    with pytest.raises(ValueError, match="int32"):
        rrs.kv_patch_lowrank(c, bt.long(), 1, [0], [8], [f])


def _decode_args(b=2, h=32, stride=4):
    return (torch.zeros((b, h, 512), dtype=BF), torch.zeros((b, h, 64), dtype=BF), mla(1), 0,
            torch.zeros((b, stride), dtype=I32), torch.zeros((b, stride), dtype=I32), torch.zeros(b, dtype=I32), 0.1)


def test_decode_checks():
    a = list(_decode_args())
    with pytest.raises(ValueError, match="CUDA"):
        rrs.mla_decode_rotate_on_read(*a)
    for i, bad, msg in ((6, torch.zeros(2, dtype=torch.int64), "int32"),
                        (6, torch.zeros(1, dtype=I32), "length per sequence"),
                        (5, torch.zeros((2, 3), dtype=I32), "match block_tables"),
                        (4, torch.zeros((1, 4), dtype=I32), "row per sequence"),
                        (1, torch.zeros((2, 32, 32), dtype=BF), "q_rope"),
                        (0, torch.zeros((2, 32, 512), dtype=F32), "q_nope")):
        b = list(a)
        b[i] = bad
        with pytest.raises(ValueError, match=msg):
            rrs.mla_decode_rotate_on_read(*b)
    with pytest.raises(ValueError, match="out"):
        rrs.mla_decode_rotate_on_read(*a, out=torch.zeros((2, 32, 128), dtype=BF))
    with pytest.raises(ValueError, match="lse"):
        rrs.mla_decode_rotate_on_read(*a, lse=torch.zeros((2, 31)))


def test_gqa_decode_checks():
    c = gqa(1)
    q = torch.zeros((2, 32, 128), dtype=BF)
    bt = torch.zeros((2, 4), dtype=I32)
    lens = torch.zeros(2, dtype=I32)
    with pytest.raises(ValueError, match="CUDA"):
        rrs.gqa_decode_rotate_on_read(q, c, 0, bt, torch.zeros_like(bt), lens, 0.1)
    with pytest.raises(ValueError, match="int32"):
        rrs.gqa_decode_rotate_on_read(q, c, 0, bt, torch.zeros_like(bt), lens.long(), 0.1)
    with pytest.raises(ValueError, match="match block_tables"):
        rrs.gqa_decode_rotate_on_read(q, c, 0, bt, torch.zeros((2, 5), dtype=I32), lens, 0.1)


def test_patch_factors_checks():
    d = torch.zeros((2, 64, 64))
    om = torch.zeros((64, 32))
    with pytest.raises(ValueError, match="CUDA"):
        rrs.kamera_patch_factors(d, 4, om)
    with pytest.raises(ValueError, match="omega"):
        rrs.kamera_patch_factors(d, 4, torch.zeros((32, 32)))
    with pytest.raises(ValueError, match="U has shape"):
        rrs.kamera_patch_factors(d, 4, om, out=(torch.zeros((2, 64, 3)), torch.zeros((2, 64, 4)),
                                                torch.zeros((2, 4))))


def test_keys_checks():
    tok = torch.zeros(100, dtype=I32)
    gear = torch.zeros(16, dtype=torch.int64)
    with pytest.raises(ValueError, match="CUDA"):
        rrs.registry_chunk_keys(tok, [0, 100], gear, 1 << 56, 8, 64, 16)
    with pytest.raises(ValueError, match="shorter than the last offset"):
        rrs.registry_chunk_keys(tok, [0, 101], gear, 1 << 56, 8, 64, 16)
