"""Absorbed-MLA decode with rotate-on-read keys, float64 (test infrastructure only).

What the pages fix:

* Irminsul §2.2 and §4: the delta-rotation of the stored k_r is fused into the
  MLA attention kernel, applied while the key is loaded from HBM, so no rotated
  copy is written back.
* Irminsul §5: the claims concern the absorbed-matmul MLA form used in
  production; in that form each query head carries a 512-d latent part
  q_nope (already multiplied into the cKV space) and a 64-d q_rope part, the
  key of token t is (cKV_t, k_r_t) and the value is cKV_t itself.
* Irminsul §2.1: cKV is position-free; only k_r carries RoPE.

Readings taken where the pages are silent:

* Each logical block of the paged cache carries one pending shift delta; the
  key actually attended is k_hat_t = R(delta_blk(t)) k_r_t, recomputed here in
  float64.  Keys live in bf16 (Leyline §4.3: rotation in fp32, KV stored in
  bf16; Irminsul §2.2: the rotation feeds the bf16 attention kernel), so with
  ``round_keys`` the attended key is that exact rotation rounded to nearest
  even in bf16 -- the key the cache would hold had the shift been applied.
  Without it the key stays unrounded (used to bound the bf16 key drift).
* s_t = scale * (q_nope . cKV_t + q_rope . k_hat_t); O = sum_t softmax(s)_t cKV_t;
  LSE = natural log of sum_t exp(s_t).  A single decode query attends to every
  cached token (no mask).
"""

import numpy as np

from . import bf16, rope


def mla_decode(q_nope, q_rope, ckv, k_r, delta_tok, scale, theta, round_keys=False):
    """Decode attention for one sequence.

    q_nope [H, Dc], q_rope [H, Dr], ckv [T, Dc], k_r [T, Dr] (float64 values),
    delta_tok [T] integer pending shift of each cached token.
    Returns (O [H, Dc], LSE [H]) in float64.
    """
    q_nope = np.asarray(q_nope, dtype=np.float64)
    q_rope = np.asarray(q_rope, dtype=np.float64)
    ckv = np.asarray(ckv, dtype=np.float64)
    dr = k_r.shape[-1]
    k_hat = rope.rotate(np.asarray(k_r, dtype=np.float64), np.asarray(delta_tok), 1, dr, theta)
    if round_keys:
        k_hat = bf16.to_f64(bf16.round_rne(k_hat))
    s = scale * (q_nope @ ckv.T + q_rope @ k_hat.T)          # [H, T]
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=1, keepdims=True)
    o = (e / z) @ ckv
    lse = (m + np.log(z))[:, 0]
    return o, lse


def score_bound(q_rope, k_r, delta_tok, scale, theta):
    """Per-head bound on the score error from storing rotated keys in bf16.

    scale * 2^-8 * max_t sum_i |q_rope[h, i]| |k_hat_t,i|, with k_hat the keys
    re-rotated in float64 (half an ulp per element plus fp32 rotation error).
    """
    dr = k_r.shape[-1]
    k_hat = rope.rotate(np.asarray(k_r, dtype=np.float64), np.asarray(delta_tok), 1, dr, theta)
    return scale * 2.0 ** -8 * (np.abs(np.asarray(q_rope, dtype=np.float64)) @ np.abs(k_hat).T).max(axis=1)


def token_deltas(block_deltas, seq_len, block_size):
    """Pending shift of every token t < seq_len from the per-block table."""
    t = np.arange(seq_len)
    return np.asarray(block_deltas)[t // block_size]


# ------------------------------------------------------------- GQA decode ---
#
# Kamera §2 re-rotates the whole GQA key and hooks its correction into the
# attention kernel; Irminsul §2.2 and §4 apply the pending rotation inside
# attention, on the load path, without writing a rotated copy back.  Taken
# together for a GQA cache (Kamera's shape: KV heads of dimension d, all of K
# rotary, V position-free):
#
#   s_t = scale * q_h . (R(delta_blk(t)) k_{t, g(h)}),   g(h) = h // (H / G)
#   O_h = sum_t softmax(s)_t v_{t, g(h)},   LSE_h = ln sum_t exp(s_t)
#
# Readings: query head h reads KV head h // (H / G) (consecutive query heads
# share a KV head); the attended key is the exact rotation of the stored key
# (no rounding: the rotation is applied in attention, not stored); one decode
# query attends to every cached token.


def gqa_decode(q, k, v, delta_tok, scale, theta, kv_heads):
    """GQA decode attention for one sequence, float64.

    q [H, d]; k, v [T, G*d] (stored rows, G = kv_heads); delta_tok [T].
    Returns (O [H, d], LSE [H]).
    """
    q = np.asarray(q, dtype=np.float64)
    H, d = q.shape
    G = int(kv_heads)
    if H % G:
        raise ValueError("query heads must be a multiple of KV heads")
    grp = H // G
    k_hat = rope.rotate(np.asarray(k, dtype=np.float64), np.asarray(delta_tok), G, d, theta)
    v = np.asarray(v, dtype=np.float64)
    o = np.empty((H, d))
    lse = np.empty(H)
    for h in range(H):
        g = h // grp
        s = scale * (k_hat[:, g * d:(g + 1) * d] @ q[h])          # [T]
        m = s.max()
        e = np.exp(s - m)
        z = e.sum()
        o[h] = (e / z) @ v[:, g * d:(g + 1) * d]
        lse[h] = m + np.log(z)
    return o, lse


def gqa_score_bound(q, k, delta_tok, scale, theta, kv_heads):
    """Per-head bound on the score error of attending with bf16 operands.

    A kernel may apply R(-delta) to q instead of R(delta) to k (the same
    product, since R is orthogonal) and round that rotated query to bf16:
    each element moves by at most 2^-8 of its magnitude, so a score moves by
    at most scale * 2^-8 * max_t sum_i |(R(-delta_t) q_h)_i| |k_{t,i}|.
    """
    q = np.asarray(q, dtype=np.float64)
    H, d = q.shape
    G = int(kv_heads)
    grp = H // G
    k = np.asarray(k, dtype=np.float64)
    dt = np.asarray(delta_tok)
    out = np.empty(H)
    for h in range(H):
        g = h // grp
        qr = rope.rotate(np.broadcast_to(q[h], (len(dt), d)), -dt, 1, d, theta)   # [T, d]
        out[h] = scale * 2.0 ** -8 * (np.abs(qr) * np.abs(k[:, g * d:(g + 1) * d])).sum(axis=1).max()
    return out
