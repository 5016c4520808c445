"""Workload descriptions and seeded draws (no relocation arithmetic here).

Shapes follow the workloads the relocation path is measured on:

* MLA rows (DeepSeek-V2/V3 style): a 512-wide position-free latent cKV and a
  64-wide rotary key k_rope, RoPE base 10000, stored together as one 576-wide
  bf16 row [cKV | k_rope] (1152 bytes).
* GQA rows: K and V of 8 KV heads x 128 dims (1024 wide each), RoPE base
  500000, K and V in separate pools.

Paged pools are laid out [layer][block][row in block][width]; a contiguous
cache is a pool of one block per sequence with the identity block table.
"""

import math
from dataclasses import dataclass, field

import numpy as np

BASE_SEED = 20260601


def rng(*keys):
    """Counter-style stream: the same keys always give the same draws."""
    return np.random.default_rng([BASE_SEED] + [int(k) for k in keys])


def _to_bf16_bits(x32):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_normal(r, shape, std=1.0):
    """N(0, std^2) samples stored as bf16, returned as uint16 bit patterns."""
    return _to_bf16_bits(r.standard_normal(shape, dtype=np.float32) * np.float32(std))


def f32_normal(r, shape, std=1.0):
    return (r.standard_normal(shape, dtype=np.float64) * std).astype(np.float32)


def _slab_seed(keys):
    return int(rng(*keys).integers(0, 2 ** 62))


def _normal_slab(flat_slab, seed, std):
    import torch
    g = torch.Generator(device=flat_slab.device)
    g.manual_seed(seed)
    flat_slab.normal_(0.0, std, generator=g)


def fill_normal_(t, *keys, std=1.0, slab_elems=1 << 28):
    """Fill a device tensor with seeded N(0, std^2) values, slab by slab.

    Each slab of the flattened tensor uses its own torch generator seeded from
    (BASE_SEED, keys, slab index), so the contents do not depend on the slab
    size of earlier calls.
    """
    flat = t.view(-1)
    n = flat.numel()
    seed0 = _slab_seed(keys)
    for i, s in enumerate(range(0, n, slab_elems)):
        _normal_slab(flat[s:min(n, s + slab_elems)], seed0 + i, std)
    return t


def normal_range_(out, lo, total, *keys, std=1.0, slab_elems=1 << 28):
    """Regenerate flat elements [lo, lo + out.numel()) of what
    ``fill_normal_(t, *keys)`` writes into a tensor of ``total`` elements,
    into ``out`` (contiguous, same dtype and device as that tensor).  Each
    generator slab that overlaps the range is redrawn whole, at its own size
    and seed, into a scratch tensor and the overlap copied out."""
    import torch
    flat = out.view(-1)
    hi = lo + flat.numel()
    seed0 = _slab_seed(keys)
    i0, i1 = lo // slab_elems, -(-hi // slab_elems)
    scratch = torch.empty(min(slab_elems, total), dtype=out.dtype, device=out.device)
    for i in range(i0, i1):
        s, e = i * slab_elems, min(total, (i + 1) * slab_elems)
        tmp = scratch[: e - s]
        _normal_slab(tmp, seed0 + i, std)
        a, b = max(s, lo), min(e, hi)
        flat[a - lo:b - lo] = tmp[a - s:b - s]
    return out


@dataclass(frozen=True)
class MLA:
    n_layers: int = 61
    pf_width: int = 512
    rope_heads: int = 1
    rope_dim: int = 64
    rope_base: float = 10000.0

    @property
    def row_width(self):
        return self.pf_width + self.rope_heads * self.rope_dim


@dataclass(frozen=True)
class GQA:
    n_layers: int = 32
    heads: int = 8
    head_dim: int = 128
    rope_base: float = 500000.0

    @property
    def width(self):
        return self.heads * self.head_dim


# ---------------------------------------------------------------- splices ---

@dataclass
class SpliceWorkload:
    name: str
    shape: MLA
    n_seq: int
    capacity: int                 # slots per sequence
    block_size: int
    n_blocks: int                 # physical blocks per layer in the pool
    block_tables: np.ndarray      # int32 [n_seq, capacity // block_size]
    seq_lens: np.ndarray          # int64 [n_seq]
    directives: np.ndarray        # int64 [n_seq, 4]: s_start, s_end, r_len, mode
    seed_keys: tuple = field(default_factory=tuple)

    @property
    def blocks_per_seq(self):
        return self.capacity // self.block_size


def single_splice():
    """One layer, one contiguous sequence of 4096 slots; replace [1000, 1800)
    by a 16-slot stub (mode AMORTIZE)."""
    return SpliceWorkload(
        name="leyline_splice_1x4096", shape=MLA(n_layers=1), n_seq=1, capacity=4096,
        block_size=4096, n_blocks=1, block_tables=np.zeros((1, 1), np.int32),
        seq_lens=np.array([4096], np.int64),
        directives=np.array([[1000, 1800, 16, 0]], np.int64), seed_keys=(1,))


def batched_splice(n_seq=64, capacity=32768, n_layers=61, block_size=64,
                   s_range=(64, 8192), r_range=(8, 64), spare_blocks=0, cfg=3,
                   allow_growth=False):
    """n_seq full sequences of ``capacity`` slots, one directive each.

    |S| ~ U{s_range}, |R| ~ U{r_range}, s_start ~ U{0 .. capacity - |S|}
    (inclusive integer draws).  Block tables are a random permutation of the
    pool's blocks; ``spare_blocks`` extra blocks stay unused (canaries).
    With ``allow_growth`` the sequences start shorter than capacity so that
    |R| > |S| still fits.
    """
    r = rng(cfg, 0)
    bps = capacity // block_size
    n_blocks = n_seq * bps + spare_blocks
    perm = r.permutation(n_blocks).astype(np.int32)
    bt = perm[: n_seq * bps].reshape(n_seq, bps)
    dirs = np.zeros((n_seq, 4), np.int64)
    lens = np.zeros(n_seq, np.int64)
    for b in range(n_seq):
        s_len = int(r.integers(s_range[0], s_range[1], endpoint=True))
        r_len = int(r.integers(r_range[0], r_range[1], endpoint=True))
        n = capacity
        if allow_growth:
            n = capacity - max(0, r_len - s_len)
        s_len = min(s_len, n)
        s0 = int(r.integers(0, n - s_len, endpoint=True))
        dirs[b] = (s0, s0 + s_len, r_len, 0)
        lens[b] = n
    return SpliceWorkload(
        name=f"leyline_splice_batched_{n_seq}x{capacity}x{n_layers}",
        shape=MLA(n_layers=n_layers), n_seq=n_seq, capacity=capacity,
        block_size=block_size, n_blocks=n_blocks, block_tables=bt, seq_lens=lens,
        directives=dirs, seed_keys=(cfg,))


# ----------------------------------------------------------------- gather ---

@dataclass
class GatherWorkload:
    name: str
    shape: MLA
    lens: np.ndarray              # int64 [n]
    base_pos: np.ndarray          # int64 [n]
    p_target: np.ndarray          # int64 [n]
    dst_slots: int
    block_size: int
    n_blocks: int                 # physical pool blocks per layer
    block_table: np.ndarray       # int32 [dst_slots // block_size]
    seed_keys: tuple = field(default_factory=tuple)


def registry_gather(n_chunks=32, dst_slots=40960, n_layers=61, block_size=64,
                    pool_blocks=1024, len_range=(256, 2048), base_range=(0, 60000), cfg=2):
    """Registry entries gathered into one destination sequence.

    len ~ U{len_range} (all lengths redrawn while their sum exceeds dst_slots),
    base_pos ~ U{base_range}; the entries are laid out in a random order and
    the unused slots are split into n+1 random gaps, so targets are not block
    aligned.  The destination block table takes dst_slots/block_size distinct
    random blocks of a pool of ``pool_blocks``; the rest stay unused.
    """
    r = rng(cfg, 0)
    while True:
        lens = r.integers(len_range[0], len_range[1], size=n_chunks, endpoint=True).astype(np.int64)
        if lens.sum() <= dst_slots:
            break
    base = r.integers(base_range[0], base_range[1], size=n_chunks, endpoint=True).astype(np.int64)
    order = r.permutation(n_chunks)
    leftover = dst_slots - int(lens.sum())
    cuts = np.sort(r.integers(0, leftover, size=n_chunks, endpoint=True))
    gaps = np.diff(np.concatenate([[0], cuts, [leftover]]))        # n+1 gaps summing to leftover
    p_target = np.zeros(n_chunks, np.int64)
    pos = int(gaps[0])
    for i, c in enumerate(order):
        p_target[c] = pos
        pos += int(lens[c]) + int(gaps[i + 1])
    nbt = dst_slots // block_size
    bt = r.permutation(pool_blocks)[:nbt].astype(np.int32)
    return GatherWorkload(
        name=f"irminsul_gather_{n_chunks}x{n_layers}", shape=MLA(n_layers=n_layers),
        lens=lens, base_pos=base, p_target=p_target, dst_slots=dst_slots,
        block_size=block_size, n_blocks=pool_blocks, block_table=bt, seed_keys=(cfg,))


# ------------------------------------------------------------------ patch ---

@dataclass
class PatchWorkload:
    name: str
    shape: GQA
    chunk_len: int
    deltas: np.ndarray            # int64 [n]
    p_target: np.ndarray          # int64 [n]
    base_pos: np.ndarray          # int64 [n]  (= p_target - delta)
    dst_slots: int
    block_size: int
    n_blocks: int
    block_table: np.ndarray       # int32 [dst_slots // block_size]
    rank: int
    factor_std: float
    seed_keys: tuple = field(default_factory=tuple)


def gqa_patch(n_chunks=16, chunk_len=1024, n_layers=32, block_size=64, rank=16,
              delta_max=30000, factor_std=0.01, spare_blocks=64, cfg=4, heads=8, head_dim=128):
    """GQA chunks relocated by delta ~ U{-delta_max..delta_max} into one sequence.

    Chunk c lands on p_target = P0 + chunk_len * pi(c), with P0 = delta_max
    rounded up to whole chunks so that every source position p_target - delta
    is non-negative.
    """
    r = rng(cfg, 0)
    p0 = int(math.ceil(delta_max / chunk_len)) * chunk_len
    deltas = r.integers(-delta_max, delta_max, size=n_chunks, endpoint=True).astype(np.int64)
    order = r.permutation(n_chunks)
    p_target = (p0 + chunk_len * order).astype(np.int64)
    dst_slots = p0 + chunk_len * n_chunks
    dst_slots = int(math.ceil(dst_slots / block_size) * block_size)
    nbt = dst_slots // block_size
    n_blocks = nbt + spare_blocks
    bt = r.permutation(n_blocks)[:nbt].astype(np.int32)
    return PatchWorkload(
        name=f"kamera_gqa_patch_{n_chunks}x{chunk_len}x{n_layers}",
        shape=GQA(n_layers=n_layers, heads=heads, head_dim=head_dim), chunk_len=chunk_len,
        deltas=deltas, p_target=p_target, base_pos=p_target - deltas, dst_slots=dst_slots,
        block_size=block_size, n_blocks=n_blocks, block_table=bt, rank=rank,
        factor_std=factor_std, seed_keys=(cfg,))


# ----------------------------------------------------------------- decode ---

@dataclass
class DecodeWorkload:
    name: str
    batch: int
    ctx: int
    heads: int
    block_size: int
    n_blocks: int
    block_tables: np.ndarray      # int32 [batch, ctx // block_size]
    pending_delta: np.ndarray     # int32 [batch, ctx // block_size]
    seq_lens: np.ndarray          # int32 [batch]
    scale: float
    shape: MLA = MLA(n_layers=1)
    seed_keys: tuple = field(default_factory=tuple)


def rotate_on_read_decode(batch=32, ctx=32768, heads=128, block_size=64, delta_max=100000,
                          cfg=5, seq_lens=None, spare_blocks=0):
    """Decode over a paged MLA cache whose blocks carry a pending shift
    delta ~ U{-delta_max..delta_max}; softmax scale 1/sqrt(576)."""
    r = rng(cfg, 0)
    bps = ctx // block_size
    n_blocks = batch * bps + spare_blocks
    bt = r.permutation(n_blocks)[: batch * bps].astype(np.int32).reshape(batch, bps)
    pend = r.integers(-delta_max, delta_max, size=(batch, bps), endpoint=True).astype(np.int32)
    if seq_lens is None:
        seq_lens = np.full(batch, ctx, np.int32)
    return DecodeWorkload(
        name=f"mla_decode_rotate_on_read_b{batch}_ctx{ctx}_h{heads}", batch=batch, ctx=ctx,
        heads=heads, block_size=block_size, n_blocks=n_blocks, block_tables=bt,
        pending_delta=pend, seq_lens=np.asarray(seq_lens, np.int32),
        scale=1.0 / math.sqrt(576.0), seed_keys=(cfg,))


@dataclass
class GqaDecodeWorkload:
    name: str
    batch: int
    ctx: int
    q_heads: int
    block_size: int
    n_blocks: int
    block_tables: np.ndarray      # int32 [batch, ctx // block_size]
    pending_delta: np.ndarray     # int32 [batch, ctx // block_size]
    seq_lens: np.ndarray          # int32 [batch]
    scale: float
    shape: GQA = GQA(n_layers=1)
    seed_keys: tuple = field(default_factory=tuple)


def gqa_rotate_on_read_decode(batch=32, ctx=32768, q_heads=32, kv_heads=8, head_dim=128, block_size=64,
                              delta_max=30000, cfg=7, seq_lens=None, spare_blocks=0):
    """Decode over a paged GQA cache (K and V of kv_heads x head_dim bf16,
    RoPE base 500000, separate pools) whose blocks carry a pending shift
    delta ~ U{-delta_max..delta_max}; q_heads / kv_heads query heads share
    each KV head; softmax scale 1/sqrt(head_dim)."""
    r = rng(cfg, 0)
    bps = ctx // block_size
    n_blocks = batch * bps + spare_blocks
    bt = r.permutation(n_blocks)[: batch * bps].astype(np.int32).reshape(batch, bps)
    pend = r.integers(-delta_max, delta_max, size=(batch, bps), endpoint=True).astype(np.int32)
    if seq_lens is None:
        seq_lens = np.full(batch, ctx, np.int32)
    return GqaDecodeWorkload(
        name=f"gqa_decode_rotate_on_read_b{batch}_ctx{ctx}_h{q_heads}_kv{kv_heads}", batch=batch, ctx=ctx,
        q_heads=q_heads, block_size=block_size, n_blocks=n_blocks, block_tables=bt, pending_delta=pend,
        seq_lens=np.asarray(seq_lens, np.int32), scale=1.0 / math.sqrt(float(head_dim)),
        shape=GQA(n_layers=1, heads=kv_heads, head_dim=head_dim), seed_keys=(cfg,))


# ------------------------------------------------------ patch formation ---

@dataclass
class PatchFormationWorkload:
    name: str
    n: int                 # deficit matrices (layers x chunks x tensors)
    rows: int              # tokens of a chunk
    cols: int              # features
    rank: int              # m
    sketch: int            # columns of the random test matrix
    orders: int            # deficits averaged per matrix (orbit patch); 1 = plain formation
    energy_dirs: int
    decay: float
    noise: float
    omega: np.ndarray      # float32 [cols, sketch], N(0, 1)
    seed_keys: tuple = field(default_factory=tuple)


def patch_formation(n_layers=32, n_chunks=16, tensors=2, rows=1024, cols=1024, rank=16, sketch=32, orders=1,
                    energy_dirs=32, decay=2.0 ** -0.125, noise=1e-3, cfg=8):
    """Deficits of the GQA patch shape (per layer, chunk and tensor a
    [1024 tokens x 1024 features] matrix) with their energy in `energy_dirs`
    feature directions (singular values ~ decay^i) plus dense noise; `orders`
    deficits per matrix for the orbit patch.  The random test matrix of the
    range finder is drawn here and passed in."""
    r = rng(cfg, 0)
    omega = r.standard_normal((cols, sketch), dtype=np.float32)
    return PatchFormationWorkload(
        name=f"patch_formation_n{n_layers * n_chunks * tensors}_{rows}x{cols}_m{rank}_p{orders}",
        n=n_layers * n_chunks * tensors, rows=rows, cols=cols, rank=rank, sketch=sketch, orders=orders,
        energy_dirs=energy_dirs, decay=decay, noise=noise, omega=omega, seed_keys=(cfg,))


def deficit_batch_(out, energy_dirs, decay, noise, *keys):
    """Fill a float32 device tensor [n, rows, cols] -- or [n, orders, rows,
    cols], the deficits of one chunk under several orders -- with seeded
    synthetic deficits: (A / sqrt(rows)) diag(decay^i) (B / sqrt(cols))^T with
    Gaussian A, B (shared by a matrix's orders: the same chunk keeps its
    low-rank directions), plus N(0, noise^2 / cols) per entry (drawn per
    order).  The matrices are built in slabs on the tensor's own device
    (input synthesis, not the method)."""
    import torch
    o4 = out if out.dim() == 4 else out.unsqueeze(1)
    n, orders, rows, cols = o4.shape
    s = torch.tensor([decay ** i for i in range(energy_dirs)], dtype=torch.float32, device=out.device)
    slab = max(1, (1 << 28) // (orders * rows * cols))
    for i0 in range(0, n, slab):
        i1 = min(n, i0 + slab)
        a = torch.empty((i1 - i0, rows, energy_dirs), dtype=torch.float32, device=out.device)
        b = torch.empty((i1 - i0, cols, energy_dirs), dtype=torch.float32, device=out.device)
        fill_normal_(a, *keys, 1, i0)
        fill_normal_(b, *keys, 2, i0)
        a *= s / rows ** 0.5
        b /= cols ** 0.5
        fill_normal_(o4[i0:i1], *keys, 3, i0, std=noise / cols ** 0.5)
        o4[i0:i1] += torch.matmul(a, b.transpose(1, 2).contiguous()).unsqueeze(1)
    return out


# ---------------------------------------------------------------- keying ---

@dataclass
class KeyingWorkload:
    name: str
    tokens: np.ndarray            # int32 [n_streams, stream_len]
    gear: np.ndarray              # uint64 [vocab]
    threshold: int                # boundary when the Gear hash is below it
    min_len: int
    max_len: int
    s1_window: int
    seed: int = 0


def registry_streams(n_streams=64, stream_len=32768, vocab=131072, n_docs=48, doc_range=(512, 4096),
                     threshold=1 << 56, min_len=64, max_len=2048, s1_window=128, cfg=6):
    """Token-id streams for registry keying.  Each stream is a random prefix
    of U{0..2047} tokens followed by documents drawn from a shared library of
    n_docs (lengths U{doc_range}), each preceded by a random run of U{0..63}
    tokens, cut at stream_len: the same content recurs at different offsets.
    Token ids are uniform over the vocabulary; the Gear table is 64-bit
    uniform per token id."""
    r = rng(cfg, 0)
    gear = r.integers(0, 2 ** 64, size=vocab, dtype=np.uint64)
    docs = [r.integers(0, vocab, size=int(r.integers(doc_range[0], doc_range[1], endpoint=True)))
            for _ in range(n_docs)]
    out = np.empty((n_streams, stream_len), np.int32)
    for s in range(n_streams):
        parts = [r.integers(0, vocab, size=int(r.integers(0, 2047, endpoint=True)))]
        n = len(parts[0])
        while n < stream_len:
            sep = r.integers(0, vocab, size=int(r.integers(0, 63, endpoint=True)))
            d = docs[int(r.integers(0, n_docs))]
            parts += [sep, d]
            n += len(sep) + len(d)
        out[s] = np.concatenate(parts)[:stream_len]
    return KeyingWorkload(name=f"registry_keying_{n_streams}x{stream_len}", tokens=out, gear=gear,
                          threshold=threshold, min_len=min_len, max_len=max_len, s1_window=s1_window)
