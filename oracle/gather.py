"""Relocating gather of registry chunks, float64 (test infrastructure only).

What the pages fix:

* Irminsul §2.2: a registry maps a content hash to a stored entry
  (cKV, k_r, base_pos).  On a hit the system takes delta = p_target - p_source,
  reuses the stored cKV as is and applies R(delta) to the stored k_r so that it
  carries the key of the new location.
* Irminsul §2.1: cKV (512-d) is position-free and needs no correction; only the
  64-d k_r slice does.
* Kamera §2: in GQA the whole K is re-rotated and V is position-free.

Readings taken where the pages are silent:

* An entry supplies ``len`` consecutive token rows; row t lands on destination
  logical slot p_target + t (all layers), written through the destination's
  block table.
* Destination ranges of the entries gathered together must not overlap; an
  overlapping request is an error (two sources for one slot).
* delta = 0 is the identity (pure copy, bit-exact rotary band too).
"""

import numpy as np

from . import rope
from .splice import decode_rope


def ranges_overlap(p_targets, lens):
    """True if any two half-open ranges [p_targets[i], p_targets[i] + lens[i]) intersect.

    Written as the plain pairwise definition; empty ranges intersect nothing.
    """
    n = len(p_targets)
    for a in range(n):
        for b in range(a + 1, n):
            if lens[a] == 0 or lens[b] == 0:
                continue
            lo = max(p_targets[a], p_targets[b])
            hi = min(p_targets[a] + lens[a], p_targets[b] + lens[b])
            if lo < hi:
                return True
    return False


def relocate_rows(pf_rows, rope_words, delta, heads, dim, theta, rope_is_bf16=True):
    """One entry's rows as they must appear at the destination.

    Returns (pf_bits, rope_ref float64, pair_norm, rotated flag).  The
    position-free words are returned untouched (bit-exact copy); the rotary
    band is R(delta) applied in float64 to the decoded stored values.
    """
    vals = decode_rope(rope_words, rope_is_bf16)
    norm = rope.pair_norms(vals, heads, dim)
    if delta == 0:
        return np.array(pf_rows), vals, norm, False
    return np.array(pf_rows), rope.rotate(vals, delta, heads, dim, theta), norm, True


def chunk_delta(p_target, base_pos):
    """delta = p_target - p_source for a registry hit (Irminsul §2.2)."""
    return int(p_target) - int(base_pos)
