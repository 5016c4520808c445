"""Shared helpers for the parity tests: host-side cache images, device
upload, and element-by-element comparison of a device result with the oracle.

Cache images are numpy arrays of raw words per layer: pf [L, rows, pf_w]
(uint16 for bf16, uint32 for f32) and rope [L, rows, rope_w] (uint16 bf16 or
float32), rows = n_blocks * block_size in physical order.
"""

from dataclasses import dataclass

import numpy as np

import kvsynth
from oracle import gather as ogather
from oracle import rope as orope
from oracle import splice as osplice
from oracle import tolerance

SENTINEL = 0x7FA5          # a NaN payload: canary rows are recognisable and bit-compared


@dataclass
class Layout:
    pf_width: int = 512
    rope_heads: int = 1
    rope_dim: int = 64
    rope_base: float = 10000.0
    rope_f32: bool = False
    interleaved: bool = True      # MLA row [pf | rope] in one bf16 pool

    @property
    def rope_width(self):
        return self.rope_heads * self.rope_dim

    def theta(self):
        return orope.inv_freq(self.rope_dim, self.rope_base)


MLA = Layout()
GQA = Layout(pf_width=1024, rope_heads=8, rope_dim=128, rope_base=500000.0, interleaved=False)
MLA_F32 = Layout(rope_f32=True, interleaved=False)


def random_image(lay, n_layers, rows, keys, special=False):
    """Seeded cache image; ``special`` sprinkles NaN/Inf/-0/subnormal words into pf."""
    r = kvsynth.rng(*keys)
    pf = kvsynth.bf16_normal(r, (n_layers, rows, lay.pf_width))
    if special:
        m = r.random(pf.shape) < 0.02
        pats = np.array([0x7FC1, 0xFFC3, 0x7F80, 0xFF80, 0x8000, 0x0001, 0x807F], np.uint16)
        pf[m] = pats[r.integers(0, len(pats), m.sum())]
    if lay.rope_f32:
        rp = kvsynth.f32_normal(r, (n_layers, rows, lay.rope_width))
    else:
        rp = kvsynth.bf16_normal(r, (n_layers, rows, lay.rope_width))
    return pf, rp


def to_device(lay, pf, rp, n_blocks, block_size):
    """Upload an image; returns (KVCache, keep-alive tensors)."""
    import torch
    from rope_rotation_splice_amd import KVCache
    L = pf.shape[0]
    if lay.interleaved:
        row = np.concatenate([pf, rp], axis=-1)
        pool = torch.from_numpy(row.view(np.int16)).view(torch.bfloat16).cuda()
        pool = pool.reshape(L, n_blocks, block_size, lay.pf_width + lay.rope_width)
        c = KVCache(pool[..., :lay.pf_width], pool[..., lay.pf_width:], lay.rope_heads, lay.rope_dim, lay.rope_base)
        return c, (pool,)
    tp = torch.from_numpy(pf.view(np.int16)).view(torch.bfloat16).cuda().reshape(L, n_blocks, block_size, -1)
    if lay.rope_f32:
        tr = torch.from_numpy(rp).cuda().reshape(L, n_blocks, block_size, -1)
    else:
        tr = torch.from_numpy(rp.view(np.int16)).view(torch.bfloat16).cuda().reshape(L, n_blocks, block_size, -1)
    return KVCache(tp, tr, lay.rope_heads, lay.rope_dim, lay.rope_base), (tp, tr)


def from_device(lay, cache):
    """Read the pool back as (pf, rope) images."""
    import torch
    L = cache.n_layers
    if lay.interleaved:
        full = torch.cat([cache.pf, cache.rope], dim=-1).reshape(L, -1, lay.pf_width + lay.rope_width)
        w = full.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        return w[..., :lay.pf_width].copy(), w[..., lay.pf_width:].copy()
    pfw = cache.pf.contiguous().reshape(L, -1, lay.pf_width).view(torch.int16).cpu().numpy().view(np.uint16)
    if lay.rope_f32:
        rpw = cache.rope.contiguous().reshape(L, -1, lay.rope_width).cpu().numpy()
    else:
        rpw = cache.rope.contiguous().reshape(L, -1, lay.rope_width).view(torch.int16).cpu().numpy().view(np.uint16)
    return pfw, rpw


def rows_to_device(lay, pf, rp):
    """Rows outside the pool ([L, len, w] images) as device tensors."""
    import torch
    tp = torch.from_numpy(np.ascontiguousarray(pf).view(np.int16)).view(torch.bfloat16).cuda()
    if lay.rope_f32:
        tr = torch.from_numpy(np.ascontiguousarray(rp)).cuda()
    else:
        tr = torch.from_numpy(np.ascontiguousarray(rp).view(np.int16)).view(torch.bfloat16).cuda()
    return tp, tr


def rope_close(lay, got, ref, scale):
    if lay.rope_f32:
        return tolerance.f32_close(got, ref, scale)
    return tolerance.bf16_close(got, ref, scale)


def bits(a):
    return a.view(np.uint32) if a.dtype == np.float32 else a


class Mismatch(AssertionError):
    pass


def check_splice(lay, before, after, block_tables, block_size, seq_lens, dirs, stubs):
    """Compare a spliced pool image with the oracle, row by row.

    before/after: (pf, rope) images.  stubs: list per sequence of (pf [L, r, w],
    rope [L, r, w]) or None.  Every physical row is checked: rows a sequence
    owns up to its new length against the oracle, rows in [new_len, N) are
    don't-care, every other row must keep its bytes.
    """
    pf0, rp0 = before
    pf1, rp1 = after
    L = pf0.shape[0]
    th = lay.theta()
    dont_care = np.zeros(pf0.shape[1], bool)
    expect_pf = pf0.copy()
    expect_rb = bits(rp0).copy()
    ref = np.full(rp0.shape, np.nan)
    scale = np.zeros(rp0.shape)
    rotated_rows = np.zeros((L, pf0.shape[1]), bool)
    new_lens = []
    for b, (n, d) in enumerate(zip(seq_lens, dirs)):
        p = osplice.plan(n, d[0], d[1], d[2], int(d[3]))
        new_lens.append(p.new_len)
        if p.mode == osplice.FORGET:
            continue
        bt = block_tables[b]
        slots = np.arange(p.new_len)
        phys = osplice.physical_rows(slots, bt, block_size)
        if p.new_len < n:
            dont_care[osplice.physical_rows(np.arange(p.new_len, n), bt, block_size)] = True
        old_phys = osplice.physical_rows(np.arange(n), bt, block_size)
        for l in range(L):
            st = stubs[b] if stubs is not None else None
            ex = osplice.splice_sequence(p, pf0[l][old_phys], rp0[l][old_phys],
                                         None if st is None else st[0][l], None if st is None else st[1][l],
                                         lay.rope_heads, lay.rope_dim, th, rope_is_bf16=not lay.rope_f32)
            stub_rows = (slots >= p.s_start) & (slots < p.s_start + p.r_len)
            if st is None:
                dont_care[phys[stub_rows]] = True
            expect_pf[l][phys] = ex.pf_bits
            expect_rb[l][phys] = bits(ex.rope_bits)
            ref[l][phys] = ex.rope_ref
            scale[l][phys] = ex.pair_norm
            rotated_rows[l][phys] = ex.rotated
    # position-free words and unrotated rotary words: bit-exact
    live = ~dont_care
    bad_pf = (pf1 != expect_pf) & live[None, :, None]
    if bad_pf.any():
        l, r, c = np.argwhere(bad_pf)[0]
        raise Mismatch(f"position-free word differs at layer {l} row {r} col {c}: "
                       f"{pf1[l, r, c]:#06x} != {expect_pf[l, r, c]:#06x} ({bad_pf.sum()} words)")
    exact = live[None, :] & ~rotated_rows
    bad_rb = (bits(rp1) != expect_rb) & exact[:, :, None]
    if bad_rb.any():
        l, r, c = np.argwhere(bad_rb)[0]
        raise Mismatch(f"unrotated rotary word differs at layer {l} row {r} col {c} ({bad_rb.sum()} words)")
    rot = live[None, :] & rotated_rows
    if rot.any():
        ok = rope_close(lay, rp1[rot], ref[rot], scale[rot])
        if not ok.all():
            i = np.argwhere(~ok)[0]
            raise Mismatch(f"rotated key outside tolerance ({(~ok).sum()} of {ok.size}); first at {i}")
    return new_lens


def check_gather(lay, before, after, block_table, block_size, entries, p_targets):
    """entries: list of (pf [L, len, w], rope [L, len, w], base_pos)."""
    pf0, rp0 = before
    pf1, rp1 = after
    L = pf0.shape[0]
    th = lay.theta()
    expect_pf = pf0.copy()
    expect_rb = bits(rp0).copy()
    ref = np.full(rp0.shape, np.nan)
    scale = np.zeros(rp0.shape)
    rotated_rows = np.zeros((L, pf0.shape[1]), bool)
    for (epf, erp, base), pt in zip(entries, p_targets):
        n = epf.shape[1]
        if n == 0:
            continue
        phys = osplice.physical_rows(pt + np.arange(n), block_table, block_size)
        d = ogather.chunk_delta(pt, base)
        for l in range(L):
            opf, r_ref, norm, rotated = ogather.relocate_rows(epf[l], erp[l], d, lay.rope_heads, lay.rope_dim, th,
                                                              rope_is_bf16=not lay.rope_f32)
            expect_pf[l][phys] = opf
            if not rotated:
                expect_rb[l][phys] = bits(erp[l])
            ref[l][phys] = r_ref
            scale[l][phys] = norm
            rotated_rows[l][phys] = rotated
    bad_pf = pf1 != expect_pf
    if bad_pf.any():
        l, r, c = np.argwhere(bad_pf)[0]
        raise Mismatch(f"position-free word differs at layer {l} row {r} col {c} ({bad_pf.sum()} words)")
    bad_rb = (bits(rp1) != expect_rb) & ~rotated_rows[:, :, None]
    if bad_rb.any():
        l, r, c = np.argwhere(bad_rb)[0]
        raise Mismatch(f"unrotated rotary word differs at layer {l} row {r} col {c} ({bad_rb.sum()} words)")
    if rotated_rows.any():
        ok = rope_close(lay, rp1[rotated_rows], ref[rotated_rows], scale[rotated_rows])
        if not ok.all():
            raise Mismatch(f"rotated key outside tolerance ({(~ok).sum()} of {ok.size})")


def check_gather_patch(lay, before, after, block_table, block_size, entries, p_targets, f_rope, f_pf):
    """Gather with Kamera's patch: K_out = R(delta) K + U V^T, V_out = V + U' V'^T.

    entries: list of (pf, rope, base_pos) images; f_rope / f_pf: per entry
    (U [L, len, m], V [L, width, m]) float32 arrays, or None (no patch).
    Unpatched position-free rows must be bit-exact copies.
    """
    from oracle import bf16 as ob, patch as opatch
    pf0, rp0 = before
    pf1, rp1 = after
    L = pf0.shape[0]
    th = lay.theta()
    touched = np.zeros(pf0.shape[1], bool)
    for i, ((epf, erp, base), pt) in enumerate(zip(entries, p_targets)):
        n = epf.shape[1]
        if n == 0:
            continue
        phys = osplice.physical_rows(pt + np.arange(n), block_table, block_size)
        touched[phys] = True
        d = ogather.chunk_delta(pt, base)
        for l in range(L):
            k = ob.to_f64(erp[l])
            fr = f_rope[i] if f_rope is not None else None
            U, V = (fr[0][l], fr[1][l]) if fr is not None else (None, None)
            y = opatch.relocate_and_patch_keys(k, d, lay.rope_heads, lay.rope_dim, th, U, V)
            scale = orope.pair_norms(k, lay.rope_heads, lay.rope_dim)
            if U is not None:
                scale = scale + opatch.patch_abs_scale(U, V)
            if d == 0 and U is None:
                if not np.array_equal(rp1[l][phys], erp[l]):
                    raise Mismatch(f"entry {i} layer {l}: unrotated unpatched keys not bit-exact")
            else:
                ok = tolerance.bf16_close(rp1[l][phys], y, scale)
                if not ok.all():
                    raise Mismatch(f"entry {i} layer {l}: {(~ok).sum()} keys outside tolerance")
            fp = f_pf[i] if f_pf is not None else None
            if fp is None:
                if not np.array_equal(pf1[l][phys], epf[l]):
                    raise Mismatch(f"entry {i} layer {l}: unpatched values not bit-exact")
            else:
                v = ob.to_f64(epf[l])
                y = opatch.patch_values(v, fp[0][l], fp[1][l])
                scale = np.abs(v) + opatch.patch_abs_scale(fp[0][l], fp[1][l])
                ok = tolerance.bf16_close(pf1[l][phys], y, scale)
                if not ok.all():
                    raise Mismatch(f"entry {i} layer {l}: {(~ok).sum()} values outside tolerance")
    if not np.array_equal(pf1[:, ~touched], pf0[:, ~touched]) or \
            not np.array_equal(bits(rp1)[:, ~touched], bits(rp0)[:, ~touched]):
        raise Mismatch("rows outside the targets changed")
