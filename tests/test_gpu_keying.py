"""Parity of registry_chunk_keys (HIP, through the C ABI) with the oracle:
Gear hashes, chunk cuts, xxHash64 fingerprints and S1 windows, bit for bit."""

import numpy as np
import pytest

import kvsynth
from oracle import keying as ok

pytestmark = pytest.mark.gpu

U64 = (1 << 64) - 1


def _u(t):
    return [int(x) & U64 for x in t.reshape(-1).cpu().numpy().astype(np.int64)]


def _run(streams, gear, thr, lo, hi, s1, seed=0, with_hash=True):
    import torch
    import rope_rotation_splice_amd as rrs
    off = np.concatenate([[0], np.cumsum([len(s) for s in streams])]).tolist()
    flat = np.concatenate([np.asarray(s, np.int32) for s in streams]) if off[-1] else np.zeros(0, np.int32)
    tok = torch.from_numpy(flat).cuda() if len(flat) else torch.zeros(0, dtype=torch.int32, device="cuda")
    g = torch.from_numpy(np.asarray(gear, np.uint64).view(np.int64)).cuda()
    out = rrs.registry_chunk_keys(tok, off, g, thr, lo, hi, s1, seed=seed, with_hash=with_hash)
    torch.cuda.synchronize()
    return off, out


def _check(streams, gear, thr, lo, hi, s1, seed, off, out, check_hash=True):
    slots = -(-hi // s1)
    for s, toks in enumerate(streams):
        toks = np.asarray(toks)
        if check_hash and len(toks):
            h = ok.gear_hashes(toks, gear)
            assert _u(out["hash"][off[s]:off[s + 1]]) == h, f"stream {s}: Gear hashes"
        ends, fps, s1fp = ok.chunk_keys(toks, gear, thr, lo, hi, s1, seed)
        n = int(out["n_chunks"][s])
        assert n == len(ends), f"stream {s}: {n} chunks, oracle {len(ends)}"
        assert out["chunk_end"][s][:n].cpu().numpy().tolist() == ends, f"stream {s}: cuts"
        assert _u(out["chunk_fp"][s][:n]) == fps, f"stream {s}: fingerprints"
        got = _u(out["s1_fp"][s][:n])
        want = [w + [0] * (slots - len(w)) for w in s1fp]
        assert got == [x for w in want for x in w], f"stream {s}: S1 windows"


def test_keys_small_streams():
    import rope_rotation_splice_amd as rrs
    r = kvsynth.rng(31, 1)
    vocab = 5000
    gear = r.integers(0, 2 ** 64, size=vocab, dtype=np.uint64)
    lens = [0, 1, 63, 64, 65, 130, 1000, 5000, 257, 3]
    streams = [r.integers(0, vocab, size=n) for n in lens]
    for thr, lo, hi, s1, seed in [(1 << 58, 16, 200, 32, 0), (1 << 56, 64, 2048, 128, 7), (1 << 62, 1, 5, 3, 2 ** 64 - 1)]:
        off, out = _run(streams, gear, thr, lo, hi, s1, seed)
        assert rrs.device_errors() == 0
        _check(streams, gear, thr, lo, hi, s1, seed, off, out)


def test_keys_shared_content_aligns():
    """The same document behind two prefixes yields shared fingerprints on
    the device as in the oracle (content-defined cuts)."""
    r = kvsynth.rng(31, 2)
    gear = r.integers(0, 2 ** 64, size=50000, dtype=np.uint64)
    doc = r.integers(0, 50000, size=6000)
    streams = [np.concatenate([r.integers(0, 50000, size=333), doc]),
               np.concatenate([r.integers(0, 50000, size=1017), doc])]
    off, out = _run(streams, gear, 1 << 56, 64, 2048, 128)
    _check(streams, gear, 1 << 56, 64, 2048, 128, 0, off, out)
    fa = set(_u(out["chunk_fp"][0][:int(out["n_chunks"][0])]))
    fb = set(_u(out["chunk_fp"][1][:int(out["n_chunks"][1])]))
    assert len(fa & fb) >= len(fa) - 3


def test_keys_bad_token_flagged():
    import rope_rotation_splice_amd as rrs
    gear = np.arange(100, dtype=np.uint64)
    _run([np.array([1, 2, 300, 4] * 20)], gear, 1 << 60, 4, 64, 16)
    assert rrs.device_errors() & 16


def test_keys_full_workload_every_stream():
    """The keying workload at full size (64 streams x 32768 tokens, vocab
    131072, threshold 2^56, chunks 64..2048, S1 windows of 128), every stream
    compared with the oracle: chunk ends, chunk fingerprints, S1 windows."""
    import rope_rotation_splice_amd as rrs
    w = kvsynth.registry_streams()
    streams = list(w.tokens)
    off, out = _run(streams, w.gear, w.threshold, w.min_len, w.max_len, w.s1_window, with_hash=False)
    assert rrs.device_errors() == 0
    for s in range(len(streams)):
        sub = {k: (v[s:s + 1] if v is not None else None) for k, v in out.items()}
        _check([streams[s]], w.gear, w.threshold, w.min_len, w.max_len, w.s1_window, w.seed, [0, len(streams[s])],
               sub, check_hash=False)


def test_keys_long_chunks_and_offset_base():
    """Chunks longer than one LDS piece (forced cuts at max_len 5000 with
    hardly any candidates) and streams that start past token 0 of the
    buffer: the leading tokens, out-of-range ids among them, are not read."""
    import torch
    import rope_rotation_splice_amd as rrs
    r = kvsynth.rng(31, 3)
    vocab = 3000
    gear = r.integers(0, 2 ** 64, size=vocab, dtype=np.uint64)
    streams = [r.integers(0, vocab, size=n) for n in (12001, 4999, 5000, 7)]
    base = 37
    lead = np.full(base, vocab + 5, dtype=np.int32)
    flat = np.concatenate([lead] + [np.asarray(s, np.int32) for s in streams])
    off = (base + np.concatenate([[0], np.cumsum([len(s) for s in streams])])).tolist()
    tok = torch.from_numpy(flat).cuda()
    g = torch.from_numpy(gear.view(np.int64)).cuda()
    for thr, lo, hi, s1 in [(1 << 50, 64, 5000, 128), (1 << 57, 100, 3000, 1000), (1 << 50, 3000, 4100, 77)]:
        out = rrs.registry_chunk_keys(tok, off, g, thr, lo, hi, s1, seed=11, with_hash=True)
        torch.cuda.synchronize()
        assert rrs.device_errors() == 0
        _check(streams, gear, thr, lo, hi, s1, 11, off, out)
        if lo > 2048 or thr == 1 << 50:
            ends = out["chunk_end"][0][:int(out["n_chunks"][0])].tolist()
            assert max(e - b for b, e in zip([0] + ends[:-1], ends)) > 2048


def test_keys_long_stream_window_refill():
    """A stream of 300000 tokens: its candidate bitmask (4688 words) is
    longer than the cut walk's on-chip window, so the walk refills it."""
    import rope_rotation_splice_amd as rrs
    r = kvsynth.rng(31, 4)
    gear = r.integers(0, 2 ** 64, size=20000, dtype=np.uint64)
    streams = [r.integers(0, 20000, size=300000), r.integers(0, 20000, size=999)]
    off, out = _run(streams, gear, 1 << 56, 64, 2048, 128, with_hash=False)
    assert rrs.device_errors() == 0
    _check(streams, gear, 1 << 56, 64, 2048, 128, 0, off, out, check_hash=False)


def test_keys_table_walk_limits():
    """The cut walk's table covers at most 4096 candidates per stream: a
    stream with ~10000 candidates takes the word scan instead, one with a few
    hundred the table.  Forced two-token chunks over 40000 tokens (about
    20000 chunks) fill the walk's on-chip list of chunk ends more than twice."""
    import rope_rotation_splice_amd as rrs
    r = kvsynth.rng(31, 5)
    gear = r.integers(0, 2 ** 64, size=7000, dtype=np.uint64)
    many = [r.integers(0, 7000, size=20000), r.integers(0, 7000, size=3000)]
    off, out = _run(many, gear, 1 << 63, 1, 9, 4, seed=5, with_hash=False)
    assert rrs.device_errors() == 0
    assert int(out["n_chunks"][0]) > 4096
    _check(many, gear, 1 << 63, 1, 9, 4, 5, off, out, check_hash=False)
    forced = [r.integers(0, 7000, size=40000)]
    off, out = _run(forced, gear, 1 << 40, 1, 2, 2, seed=6, with_hash=False)
    assert rrs.device_errors() == 0
    assert int(out["n_chunks"][0]) > 2 * 8192
    _check(forced, gear, 1 << 40, 1, 2, 2, 6, off, out, check_hash=False)
