"""Host-side checks of the C ABI: the library loads, exports every declared
entry point, and rejects invalid arguments before enqueuing anything (these
calls never reach the GPU, so they run without one)."""

import ctypes
import os
import re

import pytest

from rope_rotation_splice_amd import _abi

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "kvreloc.h")

FAKE = 1 << 40          # 256-byte aligned fake device address (never dereferenced)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w ]*?[\s\*]+(\w+)\s*\([^;{}]*\)\s*;", text, flags=re.M)
    return sorted(set(names))


def test_header_functions_exported():
    lib = _abi.load()
    names = declared_functions()
    assert {"leyline_splice", "kv_relocate_gather", "kv_patch_lowrank", "mla_decode_rotate_on_read",
            "leyline_splice_lazy", "kv_relocate_gather_lazy", "registry_chunk_keys"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_abi.SIGNATURES), "binding and header disagree"


def test_status_strings():
    lib = _abi.load()
    for s in range(-8, 2):
        assert lib.kvr_status_str(s)
    assert lib.kvr_abi_version() == 1


def mla_cache(n_layers=2, block_size=64, n_blocks=16):
    c = _abi.kvr_cache()
    c.n_layers, c.block_size, c.n_blocks = n_layers, block_size, n_blocks
    c.pf_width, c.pf_dtype = 512, _abi.KVR_BF16
    c.rope_heads, c.rope_dim, c.rope_dtype, c.rope_base = 1, 64, _abi.KVR_BF16, 10000.0
    rs = 576
    c.pf = _abi.kvr_part(FAKE, n_blocks * block_size * rs, block_size * rs, rs)
    c.rope = _abi.kvr_part(FAKE + 1024, n_blocks * block_size * rs, block_size * rs, rs)
    return c


def splice(c, dirs, lens, bt_stride=8, stubs=None, ws=FAKE, ws_bytes=1 << 20):
    lib = _abi.load()
    n = len(dirs)
    D = (_abi.kvr_directive * max(1, n))(*[_abi.kvr_directive(*d, 0) for d in dirs])
    Ls = (ctypes.c_int64 * max(1, n))(*lens)
    out = (ctypes.c_int64 * max(1, n))()
    return lib.leyline_splice(ctypes.byref(c), FAKE, bt_stride, n, Ls, D, stubs, out, ws, ws_bytes, None), out


@pytest.mark.parametrize("d,n,code", [
    ((10, 5, 1, 0), 100, -2),        # s_start > s_end
    ((-1, 5, 1, 0), 100, -2),        # negative start
    ((10, 101, 1, 0), 100, -2),      # s_end beyond the sequence
    ((10, 20, -1, 0), 100, -2),      # negative replacement length
    ((10, 20, 1, 7), 100, -1),       # unknown mode
    ((10, 20, 500, 0), 100, -3),     # grows beyond bt_stride * block_size = 512 slots
    ((0, 0, 0, 0), 600, -2),         # current length beyond capacity
])
def test_splice_validation_errors(d, n, code):
    st, _ = splice(mla_cache(), [d], [n])
    assert st == code


def test_splice_bad_cache_descriptors():
    c = mla_cache()
    c.pf_width = 500                  # 1000 bytes: not a multiple of 16
    assert splice(c, [(1, 2, 1, 0)], [10])[0] == -1
    c = mla_cache()
    c.rope_dim = 63
    assert splice(c, [(1, 2, 1, 0)], [10])[0] == -1
    c = mla_cache()
    c.pf = _abi.kvr_part(FAKE + 8, 0, 0, 576)      # misaligned base
    assert splice(c, [(1, 2, 1, 0)], [10])[0] == -1
    c = mla_cache()
    c.rope_dtype = 9
    assert splice(c, [(1, 2, 1, 0)], [10])[0] == -1


def test_splice_workspace_checked():
    # Delta = -1 over 488 moved rows: chains longer than 64 bands take the
    # ticketed mover, which needs the workspace
    c = mla_cache()
    assert splice(c, [(10, 12, 1, 0)], [500], ws=None)[0] == -6
    assert splice(c, [(10, 12, 1, 0)], [500], ws=FAKE + 16)[0] == -6
    assert splice(c, [(10, 12, 1, 0)], [500], ws_bytes=8)[0] == -6


def test_forget_only_needs_no_launch():
    st, out = splice(mla_cache(), [(30, 50, 4, 1)], [100], ws=None, ws_bytes=0)
    assert st == 1 and out[0] == 30


def test_splice_workspace_query():
    lib = _abi.load()
    c = mla_cache()
    D = (_abi.kvr_directive * 2)(_abi.kvr_directive(10, 12, 1, 0, 0), _abi.kvr_directive(0, 0, 0, 0, 0))
    Ls = (ctypes.c_int64 * 2)(500, 500)
    nbytes = lib.kvr_splice_workspace_bytes(ctypes.byref(c), 2, Ls, D)
    # ticketed (Delta = -1, 488 moved rows in 32-row tiles): 2 layers x (16 move
    # + 1 stub tile) flags, one counter per (sequence, layer), 256-byte rounded
    assert nbytes == 256 + 256
    # a shift of 285 over 200 moved rows walks one band: no workspace at all
    D[0] = _abi.kvr_directive(10, 300, 5, 0, 0)
    assert lib.kvr_splice_workspace_bytes(ctypes.byref(c), 2, Ls, D) == 0


def gather(c, ents, pts, bt_len=8):
    lib = _abi.load()
    n = len(ents)
    E = (_abi.kvr_rows * max(1, n))(*ents)
    P = (ctypes.c_int64 * max(1, n))(*pts)
    return lib.kv_relocate_gather(ctypes.byref(c), FAKE, bt_len, E, P, n, None, None, None)


def rows(length, base=0):
    return _abi.kvr_rows(FAKE, length * 576, 576, FAKE + 1024, length * 576, 576, length, base)


def test_gather_validation_errors():
    c = mla_cache()
    assert gather(c, [rows(10), rows(10)], [0, 5]) == -4          # overlapping targets
    assert gather(c, [rows(10), rows(10)], [0, 10], bt_len=0) == -1
    assert gather(c, [rows(100)], [500]) == -2                     # beyond 512-slot capacity
    assert gather(c, [rows(10)], [-1]) == -2
    bad = rows(10)
    bad.pf = FAKE + 4
    assert gather(c, [bad], [0]) == -1
    assert gather(c, [rows(10, base=-(1 << 40))], [0]) == -2       # shift does not fit 32 bits


def patch(c, ranks, part=1, bt_len=8):
    lib = _abi.load()
    n = len(ranks)
    F = (_abi.kvr_lowrank * n)(*[_abi.kvr_lowrank(FAKE, 0, FAKE + 4096, 0, r, 0) for r in ranks])
    P = (ctypes.c_int64 * n)(*[64 * i for i in range(n)])
    L = (ctypes.c_int64 * n)(*[32] * n)
    return lib.kv_patch_lowrank(ctypes.byref(c), FAKE, bt_len, part, P, L, F, n, None)


def test_patch_rank_validation():
    c = mla_cache()
    # ranks must be 0 (no patch) or a multiple of 4 up to 64; these fail before any launch
    for r in (-4, 1, 5, 18, 66, 68):
        assert patch(c, [0, r]) == -1, r
    assert patch(c, [4], part=2) == -1
    assert patch(c, [4, 4], bt_len=1) == -2        # 64-slot capacity: the second item ends at 96


def lazy(dirs, lens, B=64, bt_stride=512, stubs=FAKE, freed=FAKE):
    lib = _abi.load()
    n = len(dirs)
    D = (_abi.kvr_directive * max(1, n))(*[_abi.kvr_directive(*d, 0) for d in dirs])
    Ls = (ctypes.c_int64 * max(1, n))(*lens)
    out = (ctypes.c_int64 * max(1, n))()
    st = lib.leyline_splice_lazy(B, FAKE, FAKE, bt_stride, n, Ls, D, stubs, freed, out, None)
    return st, out


@pytest.mark.parametrize("d, n, kw, code", [
    ((65, 128, 64, 0), 4096, {}, -1),                        # s_start off the block grid
    ((64, 130, 64, 0), 4096, {}, -1),                        # s_end off the grid
    ((64, 128, 65, 0), 4096, {}, -1),                        # r_len off the grid
    ((64, 128, 64, 0), 4096, {"B": 0}, -1),
    ((64, 128, 64, 0), 4096, {"bt_stride": 8193}, -1),
    ((64, 128, 64, 0), 4096, {"stubs": None}, -1),           # stubs needed
    ((64, 128, 64, 0), 4096, {"freed": None}, -1),           # freed list needed
    ((64, 128, 64, 2), 4096, {}, -1),                        # unknown mode
    ((128, 64, 64, 0), 4096, {}, -2),                        # s_start > s_end
    ((64, 128, 64, 0), 40000, {}, -2),                       # N beyond capacity 512 * 64
    ((0, 0, 128, 0), 512 * 64, {}, -3),                      # growth beyond capacity
])
def test_lazy_validation_errors(d, n, kw, code):
    st, _ = lazy([d], [n], **kw)
    assert st == code


def lazy_gather(ents, B=64, bt_stride=64, n_seq=4, tables=FAKE):
    """ents: (seq, len, base_pos, p_target[, blocks])"""
    lib = _abi.load()
    n = len(ents)
    arr = (_abi.kvr_lazy_entry * max(1, n))()
    for i, e in enumerate(ents):
        arr[i].seq, arr[i].len, arr[i].base_pos, arr[i].p_target = e[0], e[1], e[2], e[3]
        arr[i].d_blocks = e[4] if len(e) > 4 else FAKE
        arr[i].d_pend = None
    return lib.kv_relocate_gather_lazy(B, tables, tables, bt_stride, n_seq, arr, n, FAKE, None)


@pytest.mark.parametrize("ents, kw, code", [
    ([(0, 100, 0, 65)], {}, -1),                              # target off the block grid
    ([(4, 100, 0, 64)], {}, -1),                              # sequence outside the tables
    ([(-1, 100, 0, 64)], {}, -1),
    ([(0, 100, 0, 64, None)], {}, -1),                        # blocks needed
    ([(0, 100, 0, 64)], {"B": 0}, -1),
    ([(0, 100, 0, 64)], {"bt_stride": 8193}, -1),
    ([(0, 100, 0, 64)], {"tables": None}, -1),
    ([(0, -1, 0, 64)], {}, -2),                               # negative length
    ([(0, 100, 0, -64)], {}, -2),                             # negative target
    ([(0, 100, 0, 64 * 63)], {}, -2),                         # past the table (64 blocks of 64)
    ([(0, 100, 1 << 31, 0)], {}, -2),                         # shift does not fit 32 bits
    ([(0, 100, -(1 << 31), 0)], {}, -2),
    ([(0, 100, 0, 0), (0, 10, 5, 64)], {}, -4),               # both cover logical block 1
    ([(1, 129, 0, 128), (1, 64, 0, 0), (1, 64, 0, 192)], {}, -4),
])
def test_lazy_gather_validation_errors(ents, kw, code):
    assert lazy_gather(ents, **kw) == code


def test_lazy_gather_accepts_without_launch():
    # nothing to do: no entries, or only empty ones, and distinct sequences sharing block numbers
    assert lazy_gather([]) == 0
    assert lazy_gather([(0, 0, 5, 64, None), (1, 0, 7, 64, None)]) == 0


def test_lazy_forget_and_empty_need_no_launch():
    st, out = lazy([(128, 256, 64, 1)], [4096])
    assert st == 1 and out[0] == 128
    st, _ = lazy([], [])
    assert st == 0


def keys(n_streams=2, lens=(1000, 500), cap=None, p=None, ws_bytes=1 << 20, gear=FAKE, toks=FAKE):
    lib = _abi.load()
    off = [0]
    for ln in lens:
        off.append(off[-1] + ln)
    offs = (ctypes.c_int64 * len(off))(*off)
    p = p or _abi.kvr_cdc_params(1 << 56, 64, 2048, 128, 0, 0)
    cap = cap if cap is not None else max([1] + [-(-ln // max(1, p.min_len)) for ln in lens])
    return lib.registry_chunk_keys(toks, offs, n_streams, gear, 1000, ctypes.byref(p), None, FAKE, cap, FAKE,
                                   FAKE, FAKE, FAKE, ws_bytes, None)


def test_keys_validation_errors():
    P = _abi.kvr_cdc_params
    assert keys(cap=10) == -1                                       # stream 0 needs 16 chunks
    assert keys(p=P(1, 0, 10, 128, 0, 0)) == -1                     # min_len 0
    assert keys(p=P(1, 64, 32, 128, 0, 0)) == -1                    # max_len < min_len
    assert keys(p=P(1, 64, 2048, 0, 0, 0)) == -1                    # s1 window 0
    assert keys(gear=None) == -1
    assert keys(toks=None) == -1
    assert keys(lens=(1000, -5)) == -2                              # offsets decrease
    assert keys(ws_bytes=64) == -6                                  # bitmask does not fit
    assert keys(n_streams=241, lens=tuple([10] * 241)) == -7
    assert keys(n_streams=0, lens=()) == 0
    lib = _abi.load()
    assert lib.kvr_keys_workspace_bytes(1500) == 256
    assert lib.kvr_keys_workspace_bytes(64 * 32 * 3) == 3 * 256


def gqa_cache(n_layers=2, kv_heads=8, head_dim=128, block_size=64, n_blocks=16):
    c = _abi.kvr_cache()
    c.n_layers, c.block_size, c.n_blocks = n_layers, block_size, n_blocks
    w = kv_heads * head_dim
    c.pf_width, c.pf_dtype = w, _abi.KVR_BF16
    c.rope_heads, c.rope_dim, c.rope_dtype, c.rope_base = kv_heads, head_dim, _abi.KVR_BF16, 500000.0
    c.pf = _abi.kvr_part(FAKE, n_blocks * block_size * w, block_size * w, w)
    c.rope = _abi.kvr_part(FAKE + (1 << 30), n_blocks * block_size * w, block_size * w, w)
    return c


def gqa_decode(c, batch=2, q_heads=32, layer=0, bt_stride=8, max_len=512, ws_bytes=1 << 24, q=FAKE, scale=0.1):
    lib = _abi.load()
    return lib.gqa_decode_rotate_on_read(q, batch, q_heads, ctypes.byref(c), layer, FAKE, FAKE, bt_stride, FAKE,
                                         max_len, scale, FAKE, FAKE, FAKE, ws_bytes, None)


def test_gqa_decode_validation_errors():
    lib = _abi.load()
    assert gqa_decode(gqa_cache(), q_heads=30) == -7                 # not a multiple of the KV heads
    assert gqa_decode(gqa_cache(), q_heads=8 * 17) == -7             # 17 query heads per KV head
    assert gqa_decode(gqa_cache(head_dim=64)) == -7                  # head dimension other than 128
    assert gqa_decode(gqa_cache(block_size=32)) == -7
    assert gqa_decode(gqa_cache(), layer=2) == -2
    assert gqa_decode(gqa_cache(), max_len=8 * 64 + 1) == -2         # beyond the table
    assert gqa_decode(gqa_cache(), q=FAKE + 8) == -1                 # misaligned q
    assert gqa_decode(gqa_cache(), scale=float("nan")) == -1
    assert gqa_decode(gqa_cache(), ws_bytes=16) == -6
    need = lib.kvr_gqa_decode_workspace_bytes(2, 32, 8, 512)
    assert need > 0 and lib.kvr_gqa_decode_workspace_bytes(2, 30, 8, 512) == 0
    assert gqa_decode(gqa_cache(), ws_bytes=need - 1) == -6


def form(n=2, orders=1, rows=128, cols=192, rank=16, ws_bytes=1 << 30, d=FAKE, omega=FAKE):
    lib = _abi.load()
    return lib.kamera_patch_factors(d, n, orders, rows, cols, rank, omega, FAKE, FAKE, FAKE, FAKE, ws_bytes, None)


def test_patch_factors_validation_errors():
    lib = _abi.load()
    assert form(rank=0) == -7 and form(rank=17) == -7
    assert form(rows=100) == -7 and form(cols=32) == -7 and form(rows=16384 + 64) == -7
    assert form(n=-1) == -1 and form(orders=0) == -1
    assert form(d=None) == -1 and form(omega=FAKE + 4) == -1
    assert form(ws_bytes=64) == -6
    assert form(n=0) == 0                                            # nothing to do
    need = lib.kvr_patch_factors_workspace_bytes(2, 1, 128, 192)
    assert need == (2 * 128 * 32 * 4) + (2 * 192 * 32 * 4)
    assert lib.kvr_patch_factors_workspace_bytes(2, 4, 128, 192) == need + 2 * 128 * 192 * 4
    assert form(ws_bytes=need - 1) == -6
