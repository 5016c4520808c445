"""RoPE rotation R(p) in float64 (test infrastructure only).

What the pages fix:

* Leyline §2.2: the position-dependent key band K_pe is rotated by RoPE; when
  downstream tokens shift by Delta, the cached band is corrected in closed form
  by applying R(Delta), and because RoPE rotations compose additively
  (R(a) R(b) = R(a + b)) the result equals the key rotated from scratch at the
  new position.
* Irminsul §2.1-2.2: in MLA the positional slice k_r is 64-dimensional; on a
  registry hit the stored k_r is rotated by R(delta), delta = p_target - p_source.
* Kamera §2: in GQA the whole key is re-rotated.

What the pages leave open, and the reading taken here (the plainest one,
consistent with the "half-split pairs" RoPE of the workloads):

* Pairing: within each head of rotary dimension d (h = d/2) the pairs are
  (x_j, x_{j+h}) for j < h.
* Frequencies: theta_j = base^(-2j/d), formed in float64 (or taken from a
  caller-supplied table).
* Direction: for position p and phi = p * theta_j,
      y_j     = x_j cos(phi) - x_{j+h} sin(phi)
      y_{j+h} = x_j sin(phi) + x_{j+h} cos(phi)
  i.e. the counter-clockwise plane rotation; negative p rotates backwards.
* Angles: phi is the float64 product p * theta_j, and cos/sin are taken in
  float64 (the angle is reduced in double precision, which matters at
  |p| ~ 1e5 where a float32 angle is off by ~4e-3 rad).
* Heads: every head of a multi-head key is rotated independently with the
  same theta table.
"""

import numpy as np


def inv_freq(dim, base):
    """theta_j = base^(-2j/dim), j = 0 .. dim/2 - 1, in float64."""
    if dim % 2:
        raise ValueError("rotary dimension must be even")
    j = np.arange(dim // 2, dtype=np.float64)
    return np.power(np.float64(base), -2.0 * j / np.float64(dim))


def cos_sin(p, theta):
    """cos(p*theta_j), sin(p*theta_j) in float64 for integer position shift(s) p.

    ``p`` may be a scalar or an array; the result broadcasts as p[..., None] * theta.
    """
    p = np.asarray(p, dtype=np.float64)
    phi = p[..., None] * np.asarray(theta, dtype=np.float64)
    return np.cos(phi), np.sin(phi)


def rotate(x, p, heads, dim, theta):
    """Apply R(p) to float64 keys ``x`` of shape [..., heads*dim].

    ``p`` broadcasts against the leading dimensions of ``x`` (one shift per row,
    or a scalar).  Returns a new float64 array of the same shape.
    """
    x = np.asarray(x, dtype=np.float64)
    h = dim // 2
    lead = x.shape[:-1]
    xs = x.reshape(lead + (heads, dim))
    c, s = cos_sin(np.broadcast_to(np.asarray(p, dtype=np.float64), lead), theta)
    c = c[..., None, :]            # same angle for every head
    s = s[..., None, :]
    lo = xs[..., :h]
    hi = xs[..., h:]
    y = np.empty_like(xs)
    y[..., :h] = lo * c - hi * s
    y[..., h:] = lo * s + hi * c
    return y.reshape(x.shape)


def pair_norms(x, heads, dim):
    """Per-element norm of the rotation pair the element belongs to.

    Returns an array shaped like ``x`` where element (j) and (j+h) of each head
    both hold sqrt(x_j^2 + x_{j+h}^2).  Used as the scale of the absolute floor
    of the key tolerance (cancellation makes |y| much smaller than the pair).
    """
    x = np.asarray(x, dtype=np.float64)
    h = dim // 2
    lead = x.shape[:-1]
    xs = x.reshape(lead + (heads, dim))
    n = np.hypot(xs[..., :h], xs[..., h:])
    return np.concatenate([n, n], axis=-1).reshape(x.shape)
