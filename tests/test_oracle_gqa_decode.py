"""Pins of oracle.decode's GQA form: torch's scaled_dot_product_attention on
keys rotated by an independent (complex-exponential) RoPE, a brute-force
per-key loop, a needle that only the correctly rotated key retrieves, a
grouping mutant that the library comparison rejects, and the bf16-query
score bound."""

import math

import numpy as np
import pytest
import torch

from oracle import bf16, decode, rope, tolerance


def _rot_complex(k, p, th):
    """R(p) on one head's key by complex multiplication (independent of oracle.rope)."""
    h = k.shape[-1] // 2
    z = (k[..., :h] + 1j * k[..., h:]) * np.exp(1j * np.asarray(p, dtype=np.float64)[..., None] * th)
    return np.concatenate([z.real, z.imag], axis=-1)


def _sdpa(q, k_hat, v, scale, kv_heads):
    """torch SDPA (float64, CPU) with KV heads repeated per query group."""
    H, d = q.shape
    grp = H // kv_heads
    T = k_hat.shape[0]
    K = torch.from_numpy(k_hat.reshape(T, kv_heads, d).transpose(1, 0, 2).copy()).repeat_interleave(grp, 0)
    V = torch.from_numpy(v.reshape(T, kv_heads, d).transpose(1, 0, 2).copy()).repeat_interleave(grp, 0)
    Q = torch.from_numpy(q[:, None, :].copy())
    o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, scale=scale)[:, 0, :].numpy()
    s = torch.einsum("hd,htd->ht", Q[:, 0, :], K).numpy() * scale
    lse = np.log(np.exp(s - s.max(axis=1, keepdims=True)).sum(axis=1)) + s.max(axis=1)
    return o, lse


def _rotated_keys(k, dt, kv_heads, d, th):
    T = k.shape[0]
    return np.concatenate([_rot_complex(k[:, g * d:(g + 1) * d], dt, th) for g in range(kv_heads)], axis=1).reshape(T, -1)


@pytest.mark.parametrize("H,G", [(8, 2), (32, 8), (6, 6), (16, 1)])
def test_gqa_decode_matches_sdpa_on_rotated_keys(H, G):
    r = np.random.default_rng(40 + H + G)
    d, T = 16, 200
    th = rope.inv_freq(d, 500000.0)
    q = r.standard_normal((H, d))
    k = r.standard_normal((T, G * d))
    v = r.standard_normal((T, G * d))
    dt = decode.token_deltas(r.integers(-30000, 30000, size=T // 64 + 1), T, 64)
    o, lse = decode.gqa_decode(q, k, v, dt, 0.3, th, G)
    o_ref, lse_ref = _sdpa(q, _rotated_keys(k, dt, G, d, th), v, 0.3, G)
    assert np.abs(o - o_ref).max() <= 1e-12
    assert np.abs(lse - lse_ref).max() <= 1e-12


def test_gqa_decode_zero_delta_is_plain_attention():
    r = np.random.default_rng(50)
    H, G, d, T = 8, 4, 32, 77
    q, k, v = r.standard_normal((H, d)), r.standard_normal((T, G * d)), r.standard_normal((T, G * d))
    o, lse = decode.gqa_decode(q, k, v, np.zeros(T, np.int64), 0.125, rope.inv_freq(d, 500000.0), G)
    o_ref, lse_ref = _sdpa(q, k, v, 0.125, G)
    assert np.abs(o - o_ref).max() <= 1e-12 and np.abs(lse - lse_ref).max() <= 1e-12


def test_gqa_decode_against_per_key_loop():
    r = np.random.default_rng(51)
    H, G, d, T = 4, 2, 4, 7
    th = rope.inv_freq(d, 500000.0)
    q, k, v = r.standard_normal((H, d)), r.standard_normal((T, G * d)), r.standard_normal((T, G * d))
    dt = r.integers(-100000, 100000, size=T)
    o, lse = decode.gqa_decode(q, k, v, dt, 0.7, th, G)
    for h in range(H):
        g = h // (H // G)
        s = []
        for t in range(T):
            kh = _rot_complex(k[t, g * d:(g + 1) * d], dt[t], th)
            s.append(0.7 * math.fsum(q[h, i] * kh[i] for i in range(d)))
        mx = max(s)
        w = [math.exp(x - mx) for x in s]
        z = math.fsum(w)
        for c in range(d):
            assert abs(o[h, c] - math.fsum(w[t] / z * v[t, g * d + c] for t in range(T))) <= 1e-12
        assert abs(lse[h] - (mx + math.log(z))) <= 1e-12


def test_gqa_grouping_mutant_is_rejected():
    """Mapping query head h to KV head h % G (interleaved groups) instead of
    h // (H / G) changes the result beyond the decode tolerance."""
    r = np.random.default_rng(52)
    H, G, d, T = 8, 2, 16, 128
    th = rope.inv_freq(d, 500000.0)
    q = r.standard_normal((H, d)) * 2
    k = r.standard_normal((T, G * d))
    v = r.standard_normal((T, G * d))
    dt = r.integers(-1000, 1000, size=T)
    o, lse = decode.gqa_decode(q, k, v, dt, 0.5, th, G)
    perm = np.array([h % G * (H // G) + h // G for h in range(H)])   # query order the mutant would use
    k_hat = _rotated_keys(k, dt, G, d, th)
    o_mut, lse_mut = _sdpa(q[np.argsort(perm)], k_hat, v, 0.5, G)
    o_mut, lse_mut = o_mut[perm], lse_mut[perm]
    bad = ~tolerance.decode_close(o_mut, o, lse_mut, lse)
    assert bad[[h for h in range(H) if h % G != h // (H // G)]].all()


def test_gqa_needle_and_decoy():
    """A key planted so that its correctly rotated form aligns with q is
    retrieved; a decoy aligned only when unrotated wins if the shifts are
    ignored, which fails the tolerance."""
    r = np.random.default_rng(53)
    H, G, d, T = 4, 1, 128, 512
    th = rope.inv_freq(d, 500000.0)
    q = r.standard_normal((H, d))
    q[0] *= 10.0 / np.linalg.norm(q[0])
    k = r.standard_normal((T, d)) * 0.1
    v = r.standard_normal((T, d))
    dt = decode.token_deltas(r.integers(-30000, 30000, size=T // 64), T, 64)
    needle, decoy = 400, 33
    k[needle] = _rot_complex(q[0], -dt[needle], th)          # R(d) k_needle == q_0
    k[decoy] = q[0]
    o, lse = decode.gqa_decode(q, k, v, dt, 1.0, th, G)
    cos = lambda a, b: float(a @ b / np.linalg.norm(a) / np.linalg.norm(b))
    assert cos(o[0], v[needle]) > 0.9
    o0, lse0 = decode.gqa_decode(q, k, v, np.zeros(T, np.int64), 1.0, th, G)
    assert cos(o0[0], v[needle]) < 0.5
    assert not tolerance.decode_close(o0[:1], o[:1], lse0[:1], lse[:1]).any()


def test_gqa_score_bound_covers_bf16_query():
    """Rounding the back-rotated query R(-delta) q to bf16 moves every score
    by at most the bound (single-token sequences: LSE is the score)."""
    r = np.random.default_rng(54)
    d = 128
    th = rope.inv_freq(d, 500000.0)
    worst = 0.0
    for trial in range(60):
        q = r.standard_normal((2, d)) * (1 + 4 * r.random())
        k, v = r.standard_normal((1, d)), r.standard_normal((1, d))
        dt = r.integers(-30000, 30000, size=1)
        _, lse = decode.gqa_decode(q, k, v, dt, 1 / math.sqrt(d), th, 1)
        qr = rope.rotate(q, -dt[0], 1, d, th)
        s_bf = (bf16.to_f64(bf16.round_rne(qr)) @ k[0]) / math.sqrt(d)
        bound = decode.gqa_score_bound(q, k, dt, 1 / math.sqrt(d), th, 1)
        err = np.abs(s_bf - lse)
        assert (err <= bound).all()
        worst = max(worst, float((err / bound).max()))
    assert worst > 0.01          # the bound is not vacuous by orders of magnitude
