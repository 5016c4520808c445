"""Pins of the gather, patch and decode oracles, and of the page figures."""

import json
import math
import os

import numpy as np
import pytest

from oracle import bf16, decode, gather, patch, rope

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))


# ----------------------------------------------------------------- gather ---

def test_overlap_detection_against_slot_occupancy():
    r = np.random.default_rng(0)
    for _ in range(300):
        n = int(r.integers(1, 6))
        p = r.integers(0, 40, size=n)
        ln = r.integers(0, 12, size=n)
        occ = np.zeros(64, np.int64)
        for a, b in zip(p, ln):
            occ[a:a + b] += 1
        assert gather.ranges_overlap(list(p), list(ln)) == bool((occ > 1).any())


def test_delta_rule_matches_rope_from_scratch():
    """Rows cached at base_pos + t and rotated by delta = p_target - base_pos
    carry the key of position p_target + t (Irminsul §2.2)."""
    dim, base = 64, 10000.0
    th = rope.inv_freq(dim, base)
    r = np.random.default_rng(1)
    k_raw = r.standard_normal((40, dim))
    for base_pos, p_target in [(60000, 123), (0, 40704), (777, 777), (5, 30000)]:
        stored = rope.rotate(k_raw, base_pos + np.arange(40), 1, dim, th).astype(np.float32)
        d = gather.chunk_delta(p_target, base_pos)
        pf = r.integers(0, 65535, size=(40, 8)).astype(np.uint16)
        out_pf, ref, _, rotated = gather.relocate_rows(pf, stored, d, 1, dim, th, rope_is_bf16=False)
        assert np.array_equal(out_pf, pf)
        assert rotated == (d != 0)
        scratch = rope.rotate(k_raw, p_target + np.arange(40), 1, dim, th)
        assert np.max(np.abs(ref - scratch)) <= 1e-6 * np.max(np.abs(k_raw))


def test_zero_delta_is_copy():
    dim, base = 128, 500000.0
    th = rope.inv_freq(dim, base)
    w = np.random.default_rng(2).integers(0, 65535, size=(9, 8 * dim)).astype(np.uint16)
    _, ref, _, rotated = gather.relocate_rows(np.zeros((9, 1), np.uint16), w, 0, 8, dim, th)
    assert not rotated
    assert np.array_equal(bf16.round_rne(ref)[~np.isnan(ref)], w[~np.isnan(ref)])


# ------------------------------------------------------------------ patch ---

def test_lowrank_against_triple_loop_asymmetric():
    """U [T x m], V [F x m], T != F: element (t, f) = sum_k U[t,k] V[f,k]."""
    r = np.random.default_rng(3)
    T, F, m = 5, 7, 3
    U = r.standard_normal((T, m))
    V = r.standard_normal((F, m))
    got = patch.lowrank(U, V)
    assert got.shape == (T, F)
    for t in range(T):
        for f in range(F):
            assert abs(got[t, f] - sum(U[t, k] * V[f, k] for k in range(m))) <= 1e-14


def test_lowrank_shape_96x1024():
    r = np.random.default_rng(4)
    U = r.standard_normal((96, 16))
    V = r.standard_normal((1024, 16))
    got = patch.lowrank(U, V)
    assert got.shape == (96, 1024)
    for (t, f) in [(0, 0), (95, 1023), (17, 900), (64, 3)]:
        assert abs(got[t, f] - math.fsum(U[t, k] * V[f, k] for k in range(16))) <= 1e-13


def test_patch_after_rotation_and_rank0_identity():
    dim, base, heads = 128, 500000.0, 8
    th = rope.inv_freq(dim, base)
    r = np.random.default_rng(5)
    k = r.standard_normal((12, heads * dim))
    U = r.standard_normal((12, 4))
    V = r.standard_normal((heads * dim, 4))
    got = patch.relocate_and_patch_keys(k, -30000, heads, dim, th, U, V)
    assert np.allclose(got, rope.rotate(k, -30000, heads, dim, th) + U @ V.T, rtol=0, atol=1e-12)
    assert np.array_equal(patch.patch_values(k), k)
    assert np.array_equal(patch.relocate_and_patch_keys(k, 0, heads, dim, th), k)


def test_patch_memory_fraction_matches_pages():
    """fp32 factors U [T x m] and V [d x m] against bf16 K+V of a T x d segment."""
    g = GOLDEN["patch_memory"]
    T = d = 1024
    frac = lambda m: (2 * m * (T + d) * 4) / (2 * T * d * 2)      # K and V patches / K and V bytes
    assert abs(100 * frac(16) - g["rank16_percent"]) < 0.5
    assert abs(100 * frac(64) - g["rank64_percent"]) < 0.5


def test_mla_row_split_matches_pages():
    g = GOLDEN["mla_row_split"]
    w = g["ckv_dim"] + g["kr_dim"]
    assert round(100 * g["ckv_dim"] / w) == g["ckv_percent"]
    assert round(100 * g["kr_dim"] / w) == g["kr_percent"]


def test_bf16_drift_within_pages_bound():
    """Keys stored in bf16 at their source position, rotated in fp32 and stored
    in bf16 again, stay within the pages' relative-L2 drift of the key rotated
    from scratch (Leyline §4.3, Irminsul §3)."""
    dim, base = 64, 10000.0
    th = rope.inv_freq(dim, base)
    r = np.random.default_rng(6)
    k_raw = r.standard_normal((4096, dim))
    pos = np.arange(4096)
    stored = bf16.to_f64(bf16.round_rne(rope.rotate(k_raw, pos, 1, dim, th)))
    for d in (-784, 30000, 100000):
        dev = bf16.to_f64(bf16.round_rne(rope.rotate(stored, d, 1, dim, th).astype(np.float32)))
        scratch = rope.rotate(k_raw, pos + d, 1, dim, th)
        rel = np.linalg.norm(dev - scratch) / np.linalg.norm(scratch)
        assert rel <= GOLDEN["drift"]["rel_l2_bound"]


# ----------------------------------------------------------------- decode ---

def _rot_complex(k, p, th):
    h = k.shape[-1] // 2
    z = (k[:h] + 1j * k[h:]) * np.exp(1j * p * th)
    return np.concatenate([z.real, z.imag])


def test_decode_against_per_key_loop():
    r = np.random.default_rng(7)
    H, T, Dc, Dr = 3, 9, 8, 4
    th = rope.inv_freq(Dr, 10000.0)
    qn, qr = r.standard_normal((H, Dc)), r.standard_normal((H, Dr))
    ckv, kr = r.standard_normal((T, Dc)), r.standard_normal((T, Dr))
    dt = r.integers(-100000, 100000, size=T)
    scale = 0.37
    o, lse = decode.mla_decode(qn, qr, ckv, kr, dt, scale, th)
    for h in range(H):
        s = []
        for t in range(T):
            kh = _rot_complex(kr[t], dt[t], th)
            s.append(scale * (sum(qn[h, i] * ckv[t, i] for i in range(Dc)) + sum(qr[h, i] * kh[i] for i in range(Dr))))
        mx = max(s)
        w = [math.exp(v - mx) for v in s]
        z = math.fsum(w)
        for c in range(Dc):
            assert abs(o[h, c] - math.fsum(w[t] / z * ckv[t, c] for t in range(T))) <= 1e-12
        assert abs(lse[h] - (mx + math.log(z))) <= 1e-12


def test_decode_query_side_rotation_invariance():
    """q . R(d) k == (R(-d) q) . k : the rotation can be moved to the query."""
    r = np.random.default_rng(8)
    H, T, Dc, Dr = 4, 64, 16, 64
    th = rope.inv_freq(Dr, 10000.0)
    qn, qr = r.standard_normal((H, Dc)), r.standard_normal((H, Dr))
    ckv, kr = r.standard_normal((T, Dc)), r.standard_normal((T, Dr))
    d = 4242
    o1, l1 = decode.mla_decode(qn, qr, ckv, kr, np.full(T, d), 0.1, th)
    qr2 = rope.rotate(qr, -d, 1, Dr, th)
    o2, l2 = decode.mla_decode(qn, qr2, ckv, kr, np.zeros(T, np.int64), 0.1, th)
    assert np.allclose(o1, o2, atol=1e-12) and np.allclose(l1, l2, atol=1e-12)


def test_decode_constant_values():
    r = np.random.default_rng(9)
    th = rope.inv_freq(64, 10000.0)
    row = r.standard_normal(512)
    ckv = np.tile(row, (50, 1))
    o, _ = decode.mla_decode(r.standard_normal((2, 512)), r.standard_normal((2, 64)), ckv,
                             r.standard_normal((50, 64)), r.integers(-9, 9, 50), 0.05, th)
    assert np.allclose(o, row[None, :], atol=1e-12)


def test_decode_needle_and_negative_control():
    """A key planted so that its *correctly rotated* k_r aligns with q_rope is
    retrieved.  A decoy whose *unrotated* k_r aligns with q_rope wins instead
    when the pending shifts are ignored, and the output then fails the decode
    tolerance."""
    from oracle import tolerance
    r = np.random.default_rng(10)
    T, Dc, Dr = 512, 512, 64
    th = rope.inv_freq(Dr, 10000.0)
    qn = np.zeros((1, Dc))
    qr = r.standard_normal((1, Dr))
    qr *= 8.0 / np.linalg.norm(qr)
    ckv = r.standard_normal((T, Dc))
    kr = r.standard_normal((T, Dr)) * 0.1
    blk = r.integers(-100000, 100000, size=T // 64)
    dt = decode.token_deltas(blk, T, 64)
    needle, decoy = 300, 77
    kr[needle] = rope.rotate(qr[0], -dt[needle], 1, Dr, th)       # R(d) k_needle == q_rope
    kr[decoy] = qr[0]                                              # aligned only if unrotated
    o, lse = decode.mla_decode(qn, qr, ckv, kr, dt, 1.0, th)
    cos = lambda a, b: float(a @ b / np.linalg.norm(a) / np.linalg.norm(b))
    assert cos(o[0], ckv[needle]) > 0.9
    o0, lse0 = decode.mla_decode(qn, qr, ckv, kr, np.zeros(T, np.int64), 1.0, th)
    assert cos(o0[0], ckv[needle]) < 0.5
    assert not tolerance.decode_close(o0, o, lse0, lse).any()


def test_patch_tolerance_rejects_transposed_factors():
    """On a square chunk (tokens == features) a transposed patch has the right
    shape; with unit-scale factors the key tolerance still rejects it."""
    from oracle import tolerance
    r = np.random.default_rng(11)
    T = F = 256
    U = r.standard_normal((T, 16))
    V = r.standard_normal((F, 16))
    k = r.standard_normal((T, F))
    y = k + patch.lowrank(U, V)
    scale = rope.pair_norms(k, 2, 128) + patch.patch_abs_scale(U, V)
    good = bf16.round_rne(y.astype(np.float32).astype(np.float64))
    assert tolerance.bf16_close(good, y, scale).all()
    bad = bf16.round_rne((k + patch.lowrank(V, U)).astype(np.float32).astype(np.float64))
    assert not tolerance.bf16_close(bad, y, scale).all()


def test_decode_score_bound_covers_bf16_keys():
    """The score bound covers the error of storing rotated keys in bf16: a
    single-token sequence (LSE = its score) with the keys rounded after the
    float64 rotation stays within the bound of the exact LSE, and the
    round_keys reading reproduces exactly that rounded-key attention."""
    from oracle import tolerance
    r = np.random.default_rng(12)
    th = rope.inv_freq(64, 10000.0)
    for trial in range(50):
        qn, qr = r.standard_normal((4, 512)), r.standard_normal((4, 64))
        ckv, kr = r.standard_normal((1, 512)), r.standard_normal((1, 64))
        d = r.integers(-100000, 100000, size=1)
        o, lse = decode.mla_decode(qn, qr, ckv, kr, d, 0.07, th)
        k_hat = rope.rotate(kr, d, 1, 64, th)
        s_dev = 0.07 * (qn @ ckv.T + qr @ bf16.to_f64(bf16.round_rne(k_hat)).T)[:, 0]
        eps = decode.score_bound(qr, kr, d, 0.07, th)
        assert np.all(np.abs(s_dev - lse) <= eps)
        assert tolerance.decode_close(np.tile(ckv, (4, 1)), o, s_dev, lse, eps).all()
        o_r, lse_r = decode.mla_decode(qn, qr, ckv, kr, d, 0.07, th, round_keys=True)
        assert np.allclose(lse_r, s_dev, rtol=0, atol=1e-12)
