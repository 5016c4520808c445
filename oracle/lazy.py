"""Block-aligned splice as an edit of the block table and the per-block
pending shifts, float-free (test infrastructure only).

What the pages fix:

* Leyline §2.2: downstream tokens of a splice are rotated by R(Delta) and
  re-indexed; rotations compose, R(a) R(b) = R(a + b).
* Leyline §2.3: the replacement tokens are prefilled into new slots.
* Irminsul §2.2 and §4: the rotation of the stored k_r can be applied inside
  attention, on the HBM -> on-chip load path, instead of being written back.
* Leyline §5 (drift): repeated eager splices re-round the stored keys.

Reading taken (the plainest one the rest supports): when s_start, s_end and
|R| are multiples of the block size, a splice needs no data movement at all.
Each logical block of a sequence carries a pending shift delta (its stored
k_r is the key rotated to position p - delta; attention applies R(delta)).
The splice then only

* keeps logical blocks before s_start as they are,
* gives the |R| / B new logical blocks from s_start on to caller-provided
  blocks that already hold R prefilled at its final positions (delta 0),
* moves every later logical block by Delta / B and adds Delta to its
  pending shift (composition instead of a second rotation),
* reports the blocks of [s_start, s_end) as freed; entries between the new
  and the old block count become -1 (no block) with delta 0.

new_len = N + Delta as for the eager splice.

The gather counterpart (Irminsul §2.2: a registry hit reuses a chunk's KV at
a new position with delta = p_target - p_source) takes the same reading: a
registry entry kept in pool blocks, from row 0 of its first block, and placed
at a block-aligned p_target needs no data movement either.  The destination
sequence's logical blocks p_target / B .. point at the entry's blocks (which
are then shared), each with pending shift (the entry block's own pending
shift) + delta, and the ids they replace go back to the caller.
"""

import numpy as np

from . import gather, splice


def lazy_splice_tables(bt, pend, n, s_start, s_end, r_len, block_size, stub_blocks):
    """Return (new_bt, new_pend, freed, new_len) for one sequence.

    bt, pend: int arrays of equal length (the table's capacity in blocks).
    stub_blocks: r_len / block_size physical block ids holding R.
    Raises ValueError unless s_start, s_end and r_len are block multiples and
    the result fits the table (the conditions of ``splice.plan`` too).
    """
    B = int(block_size)
    if s_start % B or s_end % B or r_len % B:
        raise ValueError("lazy splice needs block-aligned s_start, s_end and r_len")
    cap = len(bt) * B
    p = splice.plan(n, s_start, s_end, r_len, splice.AMORTIZE, cap)
    bt = np.asarray(bt, dtype=np.int64)
    pend = np.asarray(pend, dtype=np.int64)
    stub_blocks = np.asarray(stub_blocks, dtype=np.int64)
    if len(stub_blocks) != r_len // B:
        raise ValueError("one stub block per B replacement slots")
    nb_old = -(-n // B)
    nb_new = -(-p.new_len // B)
    s0b, s1b, rb = s_start // B, s_end // B, r_len // B
    db = p.delta // B
    new_bt = bt.copy()
    new_pend = pend.copy()
    for k in range(max(nb_old, nb_new)):
        if k < s0b:
            continue
        if k < s0b + rb:
            new_bt[k] = stub_blocks[k - s0b]
            new_pend[k] = 0
        elif k < nb_new:
            new_bt[k] = bt[k - db]
            new_pend[k] = pend[k - db] + p.delta
        else:
            new_bt[k] = -1
            new_pend[k] = 0
    freed = bt[s0b:s1b].copy()
    return new_bt, new_pend, freed, p.new_len


def lazy_gather_tables(bt, pend, block_size, placements):
    """Return (new_bt, new_pend, replaced) for one sequence.

    bt, pend: int arrays of equal length (the table's capacity in blocks).
    placements: list of (entry_blocks, entry_pend or None, length, base_pos,
    p_target).  Entry row r sits at row r % B of entry_blocks[r // B]; its
    block owes entry_pend[r // B] (0 if None).  replaced lists, entry after
    entry, the old ids of the logical blocks each entry now covers.
    Raises ValueError for a p_target off a block boundary, a range outside
    the table, an entry with the wrong number of blocks, or two entries
    sharing a logical block.
    """
    B = int(block_size)
    bt = np.asarray(bt, dtype=np.int64)
    pend = np.asarray(pend, dtype=np.int64)
    new_bt, new_pend = bt.copy(), pend.copy()
    replaced = []
    used = set()
    for blocks, epend, length, base_pos, p_target in placements:
        length, p_target = int(length), int(p_target)
        if p_target % B or p_target < 0 or length < 0 or p_target + length > len(bt) * B:
            raise ValueError("lazy gather needs a block-aligned target inside the table")
        nb = -(-length // B)
        blocks = np.asarray(blocks, dtype=np.int64)
        if len(blocks) != nb:
            raise ValueError("one block id per B rows of the entry")
        epend = np.zeros(nb, np.int64) if epend is None else np.asarray(epend, dtype=np.int64)
        d = gather.chunk_delta(p_target, base_pos)
        k0 = p_target // B
        for k in range(nb):
            if k0 + k in used:
                raise ValueError("two entries share a logical block")
            used.add(k0 + k)
            replaced.append(int(bt[k0 + k]))
            new_bt[k0 + k] = blocks[k]
            new_pend[k0 + k] = epend[k] + d
    return new_bt, new_pend, np.array(replaced, dtype=np.int64)
