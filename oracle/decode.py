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
