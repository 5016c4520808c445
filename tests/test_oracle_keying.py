"""Pins of oracle.keying: xxHash64 against the independent xxhash library,
the Gear recurrence against its closed 64-token-window form, the chunker
against its stated rule, and content-defined alignment on shared content."""

import numpy as np
import pytest
import xxhash


from oracle import keying as ok


@pytest.mark.parametrize("seed", [0, 1, 2 ** 63 + 5, 2 ** 64 - 1])
def test_xxh64_matches_library(seed):
    r = np.random.default_rng(3)
    for n in list(range(0, 100)) + [255, 256, 257, 1000, 4099]:
        data = r.integers(0, 256, size=n, dtype=np.uint8).tobytes()
        assert ok.xxh64(data, seed) == xxhash.xxh64_intdigest(data, seed=seed), n


def test_xxh64_published_empty_value():
    assert ok.xxh64(b"", 0) == 0xEF46DB3751D8E999


def test_gear_recurrence_equals_window_sum():
    r = np.random.default_rng(4)
    gear = r.integers(0, 2 ** 64, size=1000, dtype=np.uint64)
    toks = r.integers(0, 1000, size=500)
    h = ok.gear_hashes(toks, gear)
    g = [int(gear[t]) for t in toks]
    for i in range(len(toks)):
        w = sum(g[i - k] << k for k in range(min(64, i + 1))) % (1 << 64)
        assert h[i] == w
    # tokens 64 or more steps back do not matter: same last 64 tokens, same hash
    toks2 = np.concatenate([r.integers(0, 1000, size=37), toks[-64:]])
    assert ok.gear_hashes(toks2, gear)[-1] == h[-1]


def test_cdc_rule():
    r = np.random.default_rng(5)
    gear = r.integers(0, 2 ** 64, size=4096, dtype=np.uint64)
    toks = r.integers(0, 4096, size=20000)
    thr, lo, hi = 1 << 58, 16, 200
    h = ok.gear_hashes(toks, gear)
    ends = ok.cdc_chunks(h, thr, lo, hi)
    start = 0
    for j, e in enumerate(ends):
        n = e - start
        last = j == len(ends) - 1
        assert n <= hi and (last or n >= lo)
        cand = [i for i in range(start + lo - 1, min(start + hi, len(h))) if h[i] < thr]
        if cand:
            assert e == cand[0] + 1
        else:
            assert e == min(start + hi, len(h))
        start = e
    assert ends[-1] == len(toks)
    # the mean gap between candidates is about 2^64 / thr = 64 tokens
    rate = np.mean([x < thr for x in h])
    assert abs(rate - 1 / 64) < 0.004


def test_shared_content_gets_shared_fingerprints():
    """The same document behind different prefixes is cut at the same places
    once the chunker has met a content boundary inside it (CDC)."""
    r = np.random.default_rng(6)
    gear = r.integers(0, 2 ** 64, size=50000, dtype=np.uint64)
    doc = r.integers(0, 50000, size=6000)
    a = np.concatenate([r.integers(0, 50000, size=333), doc])
    b = np.concatenate([r.integers(0, 50000, size=1017), doc])
    ka = ok.chunk_keys(a, gear, 1 << 56, 64, 2048, 128)
    kb = ok.chunk_keys(b, gear, 1 << 56, 64, 2048, 128)
    shared = set(ka[1]) & set(kb[1])
    assert len(shared) >= len(ka[1]) - 3
    # S1 windows of shared chunks agree too
    sa = {fp: s for fp, s in zip(ka[1], ka[2])}
    sb = {fp: s for fp, s in zip(kb[1], kb[2])}
    assert all(sa[f] == sb[f] for f in shared)


def test_negative_control_fixed_offsets_do_not_align():
    """Fixed 256-token chunks (what CDC replaces) share nothing across the
    two prefixes: the alignment above comes from the content rule."""
    r = np.random.default_rng(6)
    doc = r.integers(0, 50000, size=6000)
    a = np.concatenate([r.integers(0, 50000, size=333), doc])
    b = np.concatenate([r.integers(0, 50000, size=1017), doc])
    fa = {ok.xxh64(ok.token_bytes(a[i:i + 256])) for i in range(0, len(a) - 255, 256)}
    fb = {ok.xxh64(ok.token_bytes(b[i:i + 256])) for i in range(0, len(b) - 255, 256)}
    assert not (fa & fb)


def test_s1_windows_cover_chunk():
    r = np.random.default_rng(7)
    gear = r.integers(0, 2 ** 64, size=100, dtype=np.uint64)
    toks = r.integers(0, 100, size=3000)
    ends, fps, s1 = ok.chunk_keys(toks, gear, 1 << 57, 64, 1000, 128)
    start = 0
    for e, w in zip(ends, s1):
        assert len(w) == -(-(e - start) // 128)
        assert w[0] == ok.xxh64(ok.token_bytes(toks[start:min(start + 128, e)]))
        start = e
