"""Relocation plus rank-m conditioning patch, float64 (test infrastructure only).

What the pages fix (Kamera §2):

* A reused chunk B is stored as its canonical, context-free KV together with a
  rank-m factor pair (U_m, V_m) describing the conditioning it lost.
* Reuse rebuilds it as  R(delta) * KV(B | empty) + U_m V_m^T : the keys are
  re-rotated to the new position (exact algebra, no forward pass) and the
  low-rank term is added to restore the cross-chunk binding.
* For GQA the whole K is re-rotated, and both K and V receive a patch.
* The factors come from a truncated SVD of the deficit, so U is the left
  (token-side) factor and V the right (feature-side) factor.

Readings taken where the pages are silent:

* Orientation: U is [tokens x m], V is [features x m]; the patch of element
  (t, f) is sum_k U[t, k] V[f, k].  Features of a multi-head K or V row are
  flattened head-major (f = head * head_dim + dim).
* Frame: the patch is added after the rotation, unrotated, exactly as the
  operator is written (parity unpinned beyond that formula).
* Rank 0 means no patch; V is then copied bit for bit.
"""

import numpy as np

from . import rope


def lowrank(U, V):
    """sum_k U[t, k] V[f, k] in float64 -- the rank-m patch U V^T."""
    U = np.asarray(U, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    return U @ V.T


def relocate_and_patch_keys(k_vals, delta, heads, dim, theta, U=None, V=None):
    """K_out = R(delta) K_in + U V^T in float64 (Kamera §2, GQA keys)."""
    y = k_vals if delta == 0 else rope.rotate(k_vals, delta, heads, dim, theta)
    if U is not None:
        y = y + lowrank(U, V)
    return y


def patch_values(v_vals, U=None, V=None):
    """V_out = V_in + U' V'^T in float64 (Kamera §2, GQA values)."""
    v = np.asarray(v_vals, dtype=np.float64)
    if U is None:
        return v
    return v + lowrank(U, V)


def patch_abs_scale(U, V):
    """sum_k |U[t, k]| |V[f, k]| -- magnitude scale of the patch sum per element.

    Used for the absolute floor of the tolerance (the float32 accumulation of m
    products can lose up to ~m ulps of this magnitude).
    """
    return np.abs(np.asarray(U, dtype=np.float64)) @ np.abs(np.asarray(V, dtype=np.float64)).T
