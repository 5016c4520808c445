"""Pins of the oracle's bf16 encode/decode against torch's conversion."""

import numpy as np
import torch

from oracle import bf16


def _torch_bits(x32):
    t = torch.from_numpy(np.asarray(x32, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_all_codes_round_trip():
    codes = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = bf16.to_f64(codes)
    back = bf16.round_rne(vals)
    nan = np.isnan(vals)
    assert np.array_equal(back[~nan], codes[~nan])
    assert np.all(np.isnan(bf16.to_f64(back[nan])))


def test_rne_matches_torch_on_float32_inputs():
    r = np.random.default_rng(7)
    x = np.concatenate([
        r.standard_normal(200000).astype(np.float32),
        (r.standard_normal(20000) * 1e-39).astype(np.float32),      # subnormal range
        np.clip(r.standard_normal(20000) * 3e38, -3.4e38, 3.4e38).astype(np.float32),  # near overflow
        np.array([0.0, -0.0, np.inf, -np.inf], np.float32),
    ])
    # exact midpoints between neighbouring bf16 values: ties must go to even
    codes = r.integers(0, 0x7F7F, size=20000).astype(np.uint32)
    lo = (codes << 16).view(np.float32)
    mid = (((codes << 16) | 0x8000).astype(np.uint32)).view(np.float32)
    x = np.concatenate([x, mid, -mid, lo])
    x = x[np.isfinite(x) | np.isinf(x)]
    ours = bf16.round_rne(x.astype(np.float64))
    assert np.array_equal(ours, _torch_bits(x))


def test_ties_to_even_examples():
    one = 1.0
    assert bf16.round_rne(one + 2.0 ** -8) == 0x3F80            # tie -> even (1.0)
    assert bf16.round_rne(one + 3 * 2.0 ** -8) == 0x3F82        # tie -> even (1 + 2^-6)
    assert bf16.round_rne(one + 2.0 ** -8 + 2.0 ** -30) == 0x3F81


def test_spacing_is_distance_to_next_code():
    r = np.random.default_rng(3)
    codes = r.integers(0x0080, 0x7F7F, size=5000).astype(np.uint16)   # positive normals
    v = bf16.to_f64(codes)
    nxt = bf16.to_f64(codes + np.uint16(1))
    assert np.array_equal(bf16.spacing(v), nxt - v)
    assert bf16.spacing(1.0) == 2.0 ** -7
    assert bf16.spacing(0.0) == 2.0 ** -133
