"""Kamera patch formation: the rank-m factors of a conditioning deficit, and
the orbit patch (test infrastructure only; float64).

What the pages fix (Kamera §2 and §3):

* The deficit of a chunk B reused after A is Delta = KV(B|A) - KV(B|empty), a
  [tokens x features] matrix per (layer, tensor); it is diffuse in tokens
  but low-rank in features (its energy sits in about 32 directions).
* The patch U_m V_m^T is formed once, from a conditioned forward pass on
  [A, B] followed by an SVD that keeps the m leading factors.
* A single orbit patch, averaged over permutations, serves every order of a
  cached set of chunks.

Readings taken where the pages are silent (the plainest ones the rest
supports):

* Factor convention: U [tokens x m] = U_m Sigma_m and V [features x m] = V_m,
  so that the patch is U V^T = the best rank-m approximation of Delta
  (Eckart-Young); these are exactly the factors the reuse operator adds
  (U [len][rank], V [width][rank]).  Singular vectors have a sign ambiguity;
  U V^T does not.
* Orbit patch: the deficits of a chunk under the P sampled orders are
  averaged first, and the rank-m factors are those of the mean deficit
  (averaging P rank-m patches would not be rank m).
* The forward pass itself needs model weights and is out of scope: deficits
  are synthetic inputs with the stated structure.
"""

import numpy as np


def truncated_factors(delta, m):
    """(U [T x m] = U_m Sigma_m, V [F x m], sigma [m]) of the best rank-m
    approximation of ``delta`` (float64 SVD)."""
    d = np.asarray(delta, dtype=np.float64)
    u, s, vt = np.linalg.svd(d, full_matrices=False)
    return u[:, :m] * s[:m], vt[:m].T.copy(), s[:m].copy()


def orbit_deficit(deltas):
    """Mean of the deficits of one chunk under P orders ([P, T, F] -> [T, F])."""
    return np.asarray(deltas, dtype=np.float64).mean(axis=0)


def patch(U, V):
    """The rank-m patch U V^T [T x F]."""
    return np.asarray(U, dtype=np.float64) @ np.asarray(V, dtype=np.float64).T


def tail_energy(delta, m):
    """sum_{i >= m} sigma_i^2: the squared Frobenius error of the best rank-m patch."""
    s = np.linalg.svd(np.asarray(delta, dtype=np.float64), compute_uv=False)
    return float((s[m:] ** 2).sum())
