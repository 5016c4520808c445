"""Registry keying of token streams: content-defined chunking with a Gear
rolling hash, xxHash64 fingerprints, and the S1 fixed-window fallback
(test infrastructure only; integers only).

What the pages fix (Irminsul §2.2):

* Chunks are cut by content, not by fixed offsets: a Gear rolling hash runs
  over 64-token windows and a chunk boundary is emitted when the hash falls
  below a threshold.
* Every chunk is identified by its xxHash64 fingerprint; the registry maps
  fingerprints to stored (cKV, k_r, base_pos).
* S1 (detect and recover): a CDC chunk that misses is subdivided into fixed
  128-token windows, each fingerprinted, to recover partial reuse.

Readings taken where the page is silent (the plainest ones the rest supports):

* Gear hash over token ids: h_i = (2 h_{i-1} + G[tok_i]) mod 2^64 with
  h_{-1} = 0 at each stream start.  A token's contribution is shifted out of
  the 64-bit state after 64 steps, which is what makes the window 64 tokens:
  h_i = sum_{k=0}^{63} G[tok_{i-k}] * 2^k mod 2^64 (terms before the stream
  start are absent).  G is a table of 64-bit values per token id, drawn by
  the caller (an input here, as every random draw of the method is).
* A candidate boundary follows token i when h_i < threshold (unsigned).  The
  threshold, and the chunk length bounds, are not on the page: with
  threshold t the mean gap between candidates is 2^64 / t tokens; a chunk
  is at least min_len tokens (the boundary's whole window lies in it when
  min_len >= 64) and at most max_len (a cut is forced there).  The chunk
  starting at p ends after the first candidate i in
  [p + min_len - 1, p + max_len - 1], else after p + max_len - 1; the last
  chunk of a stream ends at the stream's end.
* Fingerprint: xxHash64 of the chunk's token ids as little-endian 32-bit
  integers, with a given seed.  xxHash64 is written from its published
  specification (Yann Collet's XXH64 description: four lanes over 32-byte
  stripes, merge, tail, avalanche).
* S1 windows are aligned to their chunk's start (so they move with the
  content): [start + w s1, min(start + (w + 1) s1, end)).
"""

import numpy as np

MASK = (1 << 64) - 1
P1 = 11400714785074694791
P2 = 14029467366897019727
P3 = 1609587929392839161
P4 = 9650029242287828579
P5 = 2870177450012600261


def _rotl(x, r):
    return ((x << r) | (x >> (64 - r))) & MASK


def _round(acc, lane):
    acc = (acc + lane * P2) & MASK
    return (_rotl(acc, 31) * P1) & MASK


def _merge(acc, v):
    acc ^= _round(0, v)
    return (acc * P1 + P4) & MASK


def xxh64(data, seed=0):
    """xxHash64 of a bytes object (published XXH64 algorithm)."""
    n = len(data)
    seed &= MASK
    p = 0
    if n >= 32:
        v1 = (seed + P1 + P2) & MASK
        v2 = (seed + P2) & MASK
        v3 = seed
        v4 = (seed - P1) & MASK
        while p + 32 <= n:
            v1 = _round(v1, int.from_bytes(data[p:p + 8], "little"))
            v2 = _round(v2, int.from_bytes(data[p + 8:p + 16], "little"))
            v3 = _round(v3, int.from_bytes(data[p + 16:p + 24], "little"))
            v4 = _round(v4, int.from_bytes(data[p + 24:p + 32], "little"))
            p += 32
        h = (_rotl(v1, 1) + _rotl(v2, 7) + _rotl(v3, 12) + _rotl(v4, 18)) & MASK
        for v in (v1, v2, v3, v4):
            h = _merge(h, v)
    else:
        h = (seed + P5) & MASK
    h = (h + n) & MASK
    while p + 8 <= n:
        h ^= _round(0, int.from_bytes(data[p:p + 8], "little"))
        h = (_rotl(h, 27) * P1 + P4) & MASK
        p += 8
    if p + 4 <= n:
        h ^= (int.from_bytes(data[p:p + 4], "little") * P1) & MASK
        h = (_rotl(h, 23) * P2 + P3) & MASK
        p += 4
    while p < n:
        h ^= (data[p] * P5) & MASK
        h = (_rotl(h, 11) * P1) & MASK
        p += 1
    h ^= h >> 33
    h = (h * P2) & MASK
    h ^= h >> 29
    h = (h * P3) & MASK
    h ^= h >> 32
    return h


def gear_hashes(tokens, gear):
    """Rolling Gear hash after each token of one stream (Python ints)."""
    h = 0
    out = []
    for t in tokens:
        h = ((h << 1) + int(gear[int(t)])) & MASK
        out.append(h)
    return out


def cdc_chunks(hashes, threshold, min_len, max_len):
    """Chunk ends (exclusive, relative to the stream start) from the hashes."""
    n = len(hashes)
    ends = []
    start = 0
    while start < n:
        end = min(start + max_len, n)
        for i in range(start + min_len - 1, min(start + max_len, n)):
            if hashes[i] < threshold:
                end = i + 1
                break
        ends.append(end)
        start = end
    return ends


def token_bytes(tokens):
    return np.asarray(tokens, dtype="<i4").tobytes()


def chunk_keys(tokens, gear, threshold, min_len, max_len, s1_window, seed=0):
    """(ends, chunk fingerprints, S1 fingerprints per chunk) of one stream."""
    tokens = np.asarray(tokens)
    ends = cdc_chunks(gear_hashes(tokens, gear), threshold, min_len, max_len)
    fps, s1 = [], []
    start = 0
    for end in ends:
        fps.append(xxh64(token_bytes(tokens[start:end]), seed))
        s1.append([xxh64(token_bytes(tokens[w:min(w + s1_window, end)]), seed)
                   for w in range(start, end, s1_window)])
        start = end
    return ends, fps, s1
