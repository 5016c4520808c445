"""Pass/fail criteria between a device result and the float64 oracle.

Test infrastructure only.  The criteria follow the precision the pages fix:
keys are stored in bf16 and rotated in fp32 (Leyline §4.3); the position-free
part is reused byte for byte (Irminsul §2.1, Kamera §2).

* Position-free words, untouched rows, stubs, canaries: bitwise equality.
* Rotated bf16 keys: |g - y| <= one bf16 spacing at y, or, where the pair
  cancels (|y| much smaller than its rotation pair), <= 2^-20 * pair norm.
  y is the exact float64 rotation of the stored value; g is the device value.
  The device rounds twice (fp32 rotation, then bf16), so bit equality with a
  single rounding of y is not required.
* Rotated fp32 keys: |g - y| <= 1e-5 |y| + 2^-20 * pair norm.
* Patched values: the same bf16 criterion, with the floor scale increased by
  sum_k |U_tk| |V_fk| (float32 accumulation of the m products).
* Decode output rows, against the oracle on bf16 relocated keys: relative L2
  <= 2^-8, max abs <= 2^-7 * max |O_ref|, |LSE - LSE_ref| <= 2e-3 + eps_s.
  The device rounds the softmax weights to bf16 for the matrix cores (so
  elementwise 1-ulp is not reachable); 2e-3 covers them (their sum is off by
  at most ~2^-9 relative).  eps_s bounds the score error of a key that differs
  by up to an ulp per element (fp32 rotation then bf16 rounding can land one
  ulp away from the single rounding of the exact rotation): LSE is
  1-Lipschitz in the scores, and each score moves by at most
  scale * 2^-8 * sum_i |q_rope_i k_hat_t,i|.  See decode.score_bound.
"""

import numpy as np

from . import bf16

FLOOR = 2.0 ** -20


def bf16_close(g_bits, y, scale):
    """Boolean mask: bf16 words ``g_bits`` within tolerance of exact ``y``.

    ``scale`` is the floor scale (pair norm, plus the patch magnitude if any).
    NaN references (don't-care elements) always pass.
    """
    g = bf16.to_f64(g_bits)
    y = np.asarray(y, dtype=np.float64)
    err = np.abs(g - y)
    ok = (err <= bf16.spacing(y)) | (err <= FLOOR * np.asarray(scale, dtype=np.float64))
    return ok | np.isnan(y)


def f32_close(g, y, scale):
    """Boolean mask: float32 values within tolerance of exact ``y``."""
    g = np.asarray(g, dtype=np.float32).astype(np.float64)
    y = np.asarray(y, dtype=np.float64)
    ok = np.abs(g - y) <= 1e-5 * np.abs(y) + FLOOR * np.asarray(scale, dtype=np.float64)
    return ok | np.isnan(y)


def decode_close(o, o_ref, lse, lse_ref, eps_s=0.0):
    """Per-row boolean: decode output rows within the attention-level tolerance.

    ``eps_s`` (scalar or per row) is the bound on the score error caused by
    bf16 keys, from ``oracle.decode.score_bound``.
    """
    o = np.asarray(o, dtype=np.float64)
    o_ref = np.asarray(o_ref, dtype=np.float64)
    rel = np.linalg.norm(o - o_ref, axis=-1) <= 2.0 ** -8 * np.linalg.norm(o_ref, axis=-1)
    mx = np.abs(o - o_ref).max(axis=-1) <= 2.0 ** -7 * np.abs(o_ref).max(axis=-1)
    ls = np.abs(np.asarray(lse, np.float64) - np.asarray(lse_ref, np.float64)) <= 2e-3 + np.asarray(eps_s)
    return rel & mx & ls
