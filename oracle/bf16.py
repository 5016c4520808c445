"""bfloat16 encode/decode for the oracle (test infrastructure only).

The KV cache stores keys in bfloat16 while the rotation is done in higher
precision (Leyline §4.3: rotating in fp32 while the cache stays bf16 keeps the
drift small).  The oracle needs two exact operations:

* ``to_f64(bits)``: decode bf16 bit patterns (uint16) to float64 -- exact.
* ``round_rne(x)``: round float64 values to the nearest bf16, ties to even,
  returning uint16 bit patterns.  Used only to build stored keys and to state
  expectations; the GPU's fp32->bf16 rounding is never reproduced here.

bfloat16 = 1 sign bit, 8 exponent bits (bias 127, same range as float32),
7 stored significand bits.  Normal numbers have 8 significant bits, so the
spacing at |x| in [2^e, 2^(e+1)) is 2^(e-7); subnormals (|x| < 2^-126) have a
fixed spacing of 2^-133.
"""

import numpy as np

_BF16_MAX = float.fromhex("0x1.fe00000000000p+127")   # (2 - 2^-7) * 2^127


def to_f64(bits):
    """Decode bf16 bit patterns to float64 (exact)."""
    b = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):          # NaN payloads decode to NaN
        return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def spacing(x):
    """Distance between consecutive bf16 values around |x| (one bf16 ulp).

    For |x| in [2^e, 2^(e+1)) this is 2^(e-7); below 2^-126 it is 2^-133.
    For x == 0 the subnormal spacing is returned.
    """
    a = np.abs(np.asarray(x, dtype=np.float64))
    _, e = np.frexp(a)              # a = m * 2^e with m in [0.5, 1)  ->  a in [2^(e-1), 2^e)
    ulp = np.ldexp(1.0, e - 1 - 7)
    return np.where(a < 2.0 ** -126, 2.0 ** -133, ulp)


def round_rne(x):
    """Round float64 to bf16 (round to nearest, ties to even); return uint16 bits.

    The rounding is done exactly in float64: the value is scaled by a power of
    two so that one bf16 spacing becomes 1, rounded with ``np.rint`` (ties to
    even), and scaled back.  The result is then exactly representable in
    float32, whose upper 16 bits are the bf16 encoding.  NaN maps to the quiet
    NaN 0x7FC0 (sign kept), +-inf and overflow to +-inf.
    """
    x = np.asarray(x, dtype=np.float64)
    q = spacing(x)
    r = np.rint(x / q) * q          # exact: division/multiplication by a power of two
    # Values that round beyond the largest finite bf16 overflow to infinity.
    r = np.where(np.abs(r) > _BF16_MAX, np.copysign(np.inf, x), r)
    r = np.where(np.isinf(x), x, r)
    f = r.astype(np.float32)
    bits = (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if np.any(nan):
        sign = (np.signbit(x).astype(np.uint16) << np.uint16(15))
        bits = np.where(nan, np.uint16(0x7FC0) | sign, bits)
    return bits.astype(np.uint16)
