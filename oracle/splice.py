"""Leyline AMORTIZE splice on one sequence, float64 (test infrastructure only).

What the pages fix (Leyline §2.1-2.3):

* A directive D = (s_start, s_end, R, m) names a token range of the sequence, a
  replacement token sequence R and a mode m in {AMORTIZE, FORGET}.
* AMORTIZE splices in place: the replacement goes in, downstream positions are
  re-indexed, and the downstream tokens keep their position-free KV (K_nope and
  V; in MLA the cKV latent) unchanged.
* Replacing a range of length |S| by |R| tokens shifts every downstream token by
  Delta = |R| - |S|; the cached K_pe band of each downstream slot is corrected by
  R(Delta) (Leyline §2.2).
* The unchanged prefix [0, s_start) is kept as is; R is prefilled "into new
  slots" by the model before the rotation step (Leyline §2.3).
* FORGET sends the edit to an ordinary re-prefill with the prefix truncated.

Readings taken where the pages are silent:

* The range is half-open: |S| = s_end - s_start, downstream = [s_end, N).
* Downstream slot i moves to slot i + Delta, i.e. old [s_end, N) lands on
  [s_start + |R|, N + Delta), and new_len = N + Delta.
* The replacement rows are supplied already prefilled (a "stub"), at their final
  positions [s_start, s_start + |R|); they are copied, never rotated.  A missing
  stub leaves those slots for the caller.
* Delta = 0 is the identity: rows do not move and R(0) = I, so even the rotary
  band is unchanged bit for bit.
* FORGET moves no KV bytes; it reports new_len = s_start and a status telling the
  caller to re-prefill.  (Parity beyond this is unpinned: it needs a model.)
* Rows in [N + Delta, N) after a shrink are "don't care".
"""

from dataclasses import dataclass

import numpy as np

from . import bf16, rope

AMORTIZE = 0
FORGET = 1


@dataclass(frozen=True)
class Plan:
    """Integer bookkeeping of one directive on a sequence of length n."""
    n: int
    s_start: int
    s_end: int
    r_len: int
    mode: int
    delta: int          # |R| - |S|
    new_len: int        # n + delta (AMORTIZE) or s_start (FORGET)
    moved_rows: int     # n - s_end (0 for FORGET)


def plan(n, s_start, s_end, r_len, mode=AMORTIZE, capacity=None):
    """Decode a directive against the current length ``n`` (Leyline §2.1-2.2).

    Raises ValueError for a malformed directive (range outside [0, n], negative
    replacement length, unknown mode) or when the grown sequence would not fit
    ``capacity`` slots.
    """
    n, s_start, s_end, r_len = int(n), int(s_start), int(s_end), int(r_len)
    if mode not in (AMORTIZE, FORGET):
        raise ValueError("unknown directive mode")
    if not (0 <= s_start <= s_end <= n) or r_len < 0:
        raise ValueError("directive range outside the sequence")
    if mode == FORGET:
        return Plan(n, s_start, s_end, r_len, mode, 0, s_start, 0)
    delta = r_len - (s_end - s_start)
    new_len = n + delta
    if capacity is not None and new_len > capacity:
        raise ValueError("spliced sequence exceeds capacity")
    return Plan(n, s_start, s_end, r_len, mode, delta, new_len, n - s_end)


def source_of(p, x):
    """Where new logical slot ``x`` (0 <= x < new_len) comes from.

    Returns ("old", i) for an old slot i, or ("stub", k) for replacement row k.
    This is the per-slot statement of the splice: the prefix stays, the stub
    fills [s_start, s_start + |R|), and old slot i >= s_end lands on i + Delta.
    """
    if x < p.s_start:
        return ("old", x)
    if x < p.s_start + p.r_len:
        return ("stub", x - p.s_start)
    return ("old", x - p.delta)


@dataclass
class Expected:
    """Expected logical contents [new_len, ...] after a splice.

    pf_bits    : position-free words, bit-exact.
    rope_bits  : rotary words for rows that must be bit-exact (prefix, stub,
                 and every row when Delta == 0); undefined where ``rotated``.
    rope_ref   : float64 exact value of the rotary band (R(Delta) x for rotated
                 rows, the decoded input elsewhere).
    pair_norm  : per-element rotation-pair norm of the input (tolerance floor).
    rotated    : bool per row, True where the rotary band was rotated.
    """
    pf_bits: np.ndarray
    rope_bits: np.ndarray
    rope_ref: np.ndarray
    pair_norm: np.ndarray
    rotated: np.ndarray


def decode_rope(words, rope_is_bf16):
    """Stored rotary words -> float64 values."""
    if rope_is_bf16:
        return bf16.to_f64(words)
    return np.asarray(words, dtype=np.float32).astype(np.float64)


def sources(p, xs):
    """Vectorised ``source_of``: (is_stub bool array, index array) for slots ``xs``."""
    xs = np.asarray(xs, dtype=np.int64)
    is_stub = (xs >= p.s_start) & (xs < p.s_start + p.r_len)
    idx = np.where(xs < p.s_start, xs, np.where(is_stub, xs - p.s_start, xs - p.delta))
    return is_stub, idx


def splice_sequence(p, pf, rope_words, stub_pf, stub_rope, heads, dim, theta,
                    rope_is_bf16=True):
    """Expected logical rows of one sequence (one layer) after an AMORTIZE splice.

    ``pf`` [>= n, pf_w] and ``rope_words`` [>= n, heads*dim] are the logical
    rows before the splice (raw stored words).  ``stub_pf``/``stub_rope`` hold
    |R| prefilled replacement rows, or are None (those slots are then
    "don't care": ``rotated`` False and NaN references).
    """
    if p.mode != AMORTIZE:
        raise ValueError("splice_sequence is for AMORTIZE directives")
    nl = p.new_len
    xs = np.arange(nl, dtype=np.int64)
    is_stub, idx = sources(p, xs)
    old = ~is_stub
    out_pf = np.zeros((nl, pf.shape[1]), dtype=pf.dtype)
    out_rb = np.zeros((nl, rope_words.shape[1]), dtype=rope_words.dtype)
    ref = np.full(out_rb.shape, np.nan)
    norm = np.zeros(out_rb.shape)
    # old rows: position-free part verbatim; rotary part rotated when it moved
    out_pf[old] = pf[idx[old]]
    vals = decode_rope(rope_words[idx[old]], rope_is_bf16)
    norm[old] = rope.pair_norms(vals, heads, dim)
    moved = idx[old] >= p.s_end
    rotated = np.zeros(nl, dtype=bool)
    if p.delta != 0:
        rotated[np.flatnonzero(old)[moved]] = True
    r_ref = vals.copy()
    if p.delta != 0 and np.any(moved):
        r_ref[moved] = rope.rotate(vals[moved], p.delta, heads, dim, theta)
    ref[old] = r_ref
    keep = old & ~rotated
    out_rb[keep] = rope_words[idx[keep]]
    # stub rows: copied as given, never rotated
    if stub_pf is not None and np.any(is_stub):
        out_pf[is_stub] = stub_pf[idx[is_stub]]
        out_rb[is_stub] = stub_rope[idx[is_stub]]
        ref[is_stub] = decode_rope(stub_rope[idx[is_stub]], rope_is_bf16)
    return Expected(out_pf, out_rb, ref, norm, rotated)


def physical_rows(slots, block_table, block_size):
    """Logical slot -> physical pool row through a block table (paged KV)."""
    slots = np.asarray(slots, dtype=np.int64)
    bt = np.asarray(block_table, dtype=np.int64)
    return bt[slots // block_size] * block_size + slots % block_size
