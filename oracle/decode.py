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
  float64 without re-rounding.
* s_t = scale * (q_nope . cKV_t + q_rope . k_hat_t); O = sum_t softmax(s)_t cKV_t;
  LSE = natural log of sum_t exp(s_t).  A single decode query attends to every
  cached token (no mask).
"""

import numpy as np

from . import rope


def mla_decode(q_nope, q_rope, ckv, k_r, delta_tok, scale, theta):
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
    s = scale * (q_nope @ ckv.T + q_rope @ k_hat.T)          # [H, T]
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=1, keepdims=True)
    o = (e / z) @ ckv
    lse = (m + np.log(z))[:, 0]
    return o, lse


def token_deltas(block_deltas, seq_len, block_size):
    """Pending shift of every token t < seq_len from the per-block table."""
    t = np.arange(seq_len)
    return np.asarray(block_deltas)[t // block_size]
