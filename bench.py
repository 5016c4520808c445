#!/usr/bin/env python3
"""Throughput of the KV-relocation hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one call of the relocation path over one batch of synthetic,
seeded input that is resident in HBM before the timed region starts.  The
default workload is the batched in-place splice: 64 sequences of 32768 slots
of a 61-layer MLA cache (cKV 512 + k_r 64, bf16; 147 GB resident) in 64-slot
blocks under random block tables, one AMORTIZE directive per sequence (|S|
U{64..8192}, |R| U{8..64}, random s_start): every downstream row moves by
Delta = |R| - |S| and its k_r is rotated by R(Delta), then the prefilled stub
rows are copied in.  Other workloads: ``gather`` (32 registry entries
gathered into one 40960-slot paged sequence, each rotated by its own
delta = p_target - base_pos), ``splice`` (one 4096-slot contiguous sequence,
[1000, 1800) -> 16 stub slots), ``gqa_patch`` (GQA relocation with a rank-16
patch), ``decode`` (rotate-on-read MLA decode, batch 32 x 32768 tokens x 128
heads; ``decode_zero_delta`` is the same with every pending shift 0), the
lazy and keying workloads, patch formation, and ``copy`` (a plain device
copy).

Prints one JSON line: slots relocated per second (a slot = one token
position of one sequence, all layers), the roofline of the relocation
kernel (algorithmic bytes / kernel time vs 8 TB/s), and the CPU oracle timed
on the host's cores on a bounded sample of the same workload.
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "KV slots relocated/sec (δ-rotate + splice) and achieved HBM GB/s vs peak"
MLA_ROW_BYTES = 1152


# sources each kernel is built from: a change to any of them makes the stored
# HBM counters stale (the shared headers and the host side count for all)
KERNEL_SOURCES = {
    "reloc_kernel": ["relocate.hip"],
    "band_kernel": ["band.hip"],
    "patch_dma_kernel": ["patch.hip"],
    "patch_kernel": ["patch.hip"],
    "mla_decode_kernel": ["decode.hip", "kvr_lds.h"],
    "gqa_decode_kernel": ["gqa_decode.hip", "kvr_lds.h"],
    "power_kernel": ["patch_form.hip"],
}
SHARED_SOURCES = ["kvr_device.h", "kvr_internal.h", "api.cpp"]


def kernel_source_hash(kernel=None):
    """Hash of the sources of ``kernel`` (key prefix as in KERNEL_SOURCES),
    or of every source when ``kernel`` is None."""
    p = os.path.join(ROOT, "rope_rotation_splice_amd", "csrc")
    if kernel is None:
        files = sorted(f for f in os.listdir(p) if f.endswith((".hip", ".h", ".cpp")))
    else:
        own = next((v for k, v in KERNEL_SOURCES.items() if kernel.startswith(k)), None)
        files = sorted(SHARED_SOURCES + own) if own else sorted(
            f for f in os.listdir(p) if f.endswith((".hip", ".h", ".cpp")))
    h = hashlib.sha256()
    for f in files:
        h.update(f.encode())
        h.update(open(os.path.join(p, f), "rb").read())
    h.update(open(os.path.join(ROOT, "include", "kvreloc.h"), "rb").read())
    return h.hexdigest()[:16]


def stored_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 PMC summary, if it
    was taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(f"{kernel}/{workload}")
    except (ValueError, OSError):
        return None
    if not rec or rec.get("source_hash") != kernel_source_hash(kernel):
        return None
    return rec.get("traffic_bytes_per_launch")


# ------------------------------------------------------------ CPU oracle ---
#
# The oracle runs on the host's cores before the GPU is touched: a pool of
# worker processes (one per core of this process's CPU set, at most 16, the
# host share of one GPU), each with single-threaded BLAS.  Worker w takes the
# workload's oracle slabs w, w + n, w + 2n, ... (cycling when the workload has
# fewer), regenerates each slab's inputs untimed and times only the oracle
# call, until its own oracle time reaches the budget.  The reported rate is
# the sum of the workers' rates, which ran side by side.

def oracle_workers():
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _oracle_worker(spec):
    name, w, n, budget = spec
    wl = WORKLOADS[name]()
    total = wl.oracle_slabs()
    units, spent, gen, slabs = 0, 0.0, 0.0, 0
    i = w
    while spent < budget:
        u, s, g = wl.oracle_slab(i % total)
        units += u
        spent += s
        gen += g
        slabs += 1
        i += n
    return units, spent, gen, slabs


def oracle_baseline(name, budget_s, unit, what):
    """Run ``name``'s oracle slabs in a process pool; returns the cpu_baseline record."""
    import multiprocessing as mp
    n = oracle_workers()
    saved = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
    for k in saved:
        os.environ[k] = "1"
    try:
        t0 = time.perf_counter()
        with mp.get_context("spawn").Pool(n) as pool:
            res = pool.map(_oracle_worker, [(name, w, n, budget_s) for w in range(n)])
        wall = time.perf_counter() - t0
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    units = sum(r[0] for r in res)
    rate = sum(r[0] / r[1] for r in res if r[1] > 0)
    slabs = sum(r[3] for r in res)
    return {"value": rate, "unit": unit, "cores": n, "kind": "oracle",
            "sample": f"{slabs} {what} ({units:.0f} {unit.split('/')[0]}) on {n} worker processes with "
                      f"single-threaded BLAS, {budget_s:g} s of oracle time each; the rate is the sum of the "
                      f"workers' rates; input generation excluded ({sum(r[2] for r in res):.1f} s in all); "
                      f"pool wall time {wall:.1f} s",
            "oracle_s": sum(r[1] for r in res)}


# --------------------------------------------------------------- workloads ---

class Gather:
    name = "registry_gather"
    kernel = "reloc_kernel<gather>"

    def __init__(self):
        import kvsynth
        self.w = kvsynth.registry_gather()
        self.slots = int(self.w.lens.sum())
        L = self.w.shape.n_layers
        self.bytes = self.slots * L * MLA_ROW_BYTES * 2 + self.w.block_table.nbytes
        self.launches = 1
        self.config = {"workload": "irminsul_registry_gather", "layers": L, "entries": len(self.w.lens),
                       "dst_slots": self.w.dst_slots, "block_size": self.w.block_size,
                       "entry_len": "U{256..2048}", "base_pos": "U{0..60000}", "slots_per_step": self.slots,
                       "row": "cKV 512 + k_r 64 bf16", "rope_base": 10000}

    def setup(self):
        import torch
        import kvsynth
        import rope_rotation_splice_amd as rrs
        w = self.w
        L, B = w.shape.n_layers, w.block_size
        self.pool = torch.empty((L, w.n_blocks, B, 576), dtype=torch.bfloat16, device="cuda")
        kvsynth.fill_normal_(self.pool, 2, 1)
        self.cache = rrs.KVCache.mla(self.pool)
        self.ents = []
        for i, ln in enumerate(w.lens):
            ckv = torch.empty((L, int(ln), 512), dtype=torch.bfloat16, device="cuda")
            kr = torch.empty((L, int(ln), 64), dtype=torch.bfloat16, device="cuda")
            kvsynth.fill_normal_(ckv, 2, 2, i, 0)
            kvsynth.fill_normal_(kr, 2, 2, i, 1)
            self.ents.append(rrs.Rows(ckv, kr, int(w.base_pos[i])))
        self.bt = torch.from_numpy(w.block_table).cuda()
        self.pt = w.p_target.tolist()
        self.rrs = rrs

    def step(self):
        self.rrs.kv_relocate_gather(self.cache, self.bt, self.ents, self.pt)

    oracle_what = "(entry, layer) slabs of the same draw, gathered and rotated (numpy fp64)"

    def oracle_slabs(self):
        return len(self.w.lens) * self.w.shape.n_layers

    def oracle_slab(self, i):
        """One (entry, layer) slab through the oracle's gather: (slots, oracle s, generation s)."""
        import kvsynth
        from oracle import gather as og, rope as orope
        w = self.w
        L = w.shape.n_layers
        e, l = i // L, i % L
        ln = int(w.lens[e])
        t0 = time.perf_counter()
        r = kvsynth.rng(2, 9, e, l)
        pf = kvsynth.bf16_normal(r, (ln, 512))
        rp = kvsynth.bf16_normal(r, (ln, 64))
        th = orope.inv_freq(64, 10000.0)
        d = og.chunk_delta(int(w.p_target[e]), int(w.base_pos[e]))
        t1 = time.perf_counter()
        og.relocate_rows(pf, rp, d, 1, 64, th)
        t2 = time.perf_counter()
        return ln / L, t2 - t1, t1 - t0


class Splice:
    name = "single_splice"
    kernel = "band_kernel"

    def __init__(self):
        import kvsynth
        self.w = kvsynth.single_splice()
        d = self.w.directives[0]
        moved = 4096 - int(d[1])
        self.slots = moved
        self.bytes = (moved + int(d[2])) * MLA_ROW_BYTES * 2
        self.launches = 1
        self.config = {"workload": "leyline_single_splice", "layers": 1, "slots": 4096,
                       "directive": [int(d[0]), int(d[1]), int(d[2]), "AMORTIZE"], "delta": int(d[2]) - int(d[1] - d[0]),
                       "slots_per_step": moved, "layout": "contiguous"}

    def setup(self):
        import torch
        import kvsynth
        import rope_rotation_splice_amd as rrs
        self.pool = torch.empty((1, 1, 4096, 576), dtype=torch.bfloat16, device="cuda")
        kvsynth.fill_normal_(self.pool, 1, 1)
        self.stub = torch.empty((1, 16, 576), dtype=torch.bfloat16, device="cuda")
        kvsynth.fill_normal_(self.stub, 1, 2)
        self.cache = rrs.KVCache.mla(self.pool)
        self.bt = torch.zeros((1, 1), dtype=torch.int32, device="cuda")
        self.dirs = [tuple(int(x) for x in self.w.directives[0])]
        self.stubs = [rrs.Rows(self.stub[..., :512], self.stub[..., 512:])]
        self.rrs = rrs

    def step(self):
        # the same directive on the restored length: same bytes and hazards each step
        self.rrs.leyline_splice(self.cache, self.bt, [4096], self.dirs, self.stubs)

    def extra(self):
        """Latency of one call, end to end (host marshalling, launch and the
        kernel, to completion), warm and after writing 1 GiB to flush the
        L2 and the MALL: medians of 30 calls each."""
        import torch
        flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        out = {}
        for kind in ("warm", "after_1GiB_flush"):
            ts = []
            for _ in range(30):
                if kind != "warm":
                    flush.zero_()
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                self.step()
                torch.cuda.synchronize()
                ts.append((time.perf_counter() - t0) * 1e6)
            out[kind] = float(np.median(ts))
        del flush
        return {"latency_us": out}

    oracle_what = "whole single-sequence splices (numpy fp64)"

    def oracle_slabs(self):
        return 1

    def oracle_slab(self, i):
        import kvsynth
        from oracle import splice as osplice, rope as orope
        t0 = time.perf_counter()
        th = orope.inv_freq(64, 10000.0)
        d = self.w.directives[0]
        p = osplice.plan(4096, int(d[0]), int(d[1]), int(d[2]), 0)
        r = kvsynth.rng(1, 9)
        pf = kvsynth.bf16_normal(r, (4096, 512))
        rp = kvsynth.bf16_normal(r, (4096, 64))
        spf = kvsynth.bf16_normal(r, (16, 512))
        srp = kvsynth.bf16_normal(r, (16, 64))
        t1 = time.perf_counter()
        n = 0
        while n == 0 or time.perf_counter() - t1 < 0.5:
            osplice.splice_sequence(p, pf, rp, spf, srp, 1, 64, th)
            n += 1
        t2 = time.perf_counter()
        return n * self.slots, t2 - t1, t1 - t0


class SpliceBatched:
    name = "batched_splice"
    kernel = "reloc_kernel<splice>"

    def __init__(self):
        import kvsynth
        self.w = kvsynth.batched_splice()
        d = self.w.directives
        moved = (self.w.seq_lens - d[:, 1]).astype(np.int64)
        delta = d[:, 2] - (d[:, 1] - d[:, 0])
        moved = np.where(delta != 0, moved, 0)
        L = self.w.shape.n_layers
        self.slots = int(moved.sum())
        self.bytes = int((moved.sum() + d[:, 2].sum()) * L * MLA_ROW_BYTES * 2)
        self.launches = 2          # 64 sequences, 32 per launch
        self.config = {"workload": "leyline_batched_splices", "sequences": self.w.n_seq, "slots": self.w.capacity,
                       "layers": L, "block_size": self.w.block_size, "S_len": "U{64..8192}", "R_len": "U{8..64}",
                       "slots_per_step": self.slots, "resident_GB": round(self.w.n_blocks * 64 * L * 1152 / 1e9, 1)}

    def setup(self):
        import torch
        import kvsynth
        import rope_rotation_splice_amd as rrs
        w = self.w
        L = w.shape.n_layers
        self.pool = torch.empty((L, w.n_blocks, w.block_size, 576), dtype=torch.bfloat16, device="cuda")
        kvsynth.fill_normal_(self.pool, 3, 1)
        self.cache = rrs.KVCache.mla(self.pool)
        self.bt = torch.from_numpy(w.block_tables).cuda()
        self.stub_t = []
        self.stubs = []
        for b in range(w.n_seq):
            st = torch.empty((L, int(w.directives[b, 2]), 576), dtype=torch.bfloat16, device="cuda")
            kvsynth.fill_normal_(st, 3, 2, b)
            self.stub_t.append(st)
            self.stubs.append(rrs.Rows(st[..., :512], st[..., 512:]))
        self.dirs = [tuple(int(x) for x in d) for d in w.directives]
        self.lens = w.seq_lens.tolist()
        self.rrs = rrs

    def step(self):
        self.rrs.leyline_splice(self.cache, self.bt, self.lens, self.dirs, self.stubs)

    oracle_what = "(sequence, layer) slabs of the same directives, spliced and rotated (numpy fp64)"

    def oracle_slabs(self):
        return self.w.n_seq * self.w.shape.n_layers

    def oracle_slab(self, i):
        """One (sequence, layer) slab: the whole sequence through the oracle's splice."""
        import kvsynth
        from oracle import splice as osplice, rope as orope
        w = self.w
        b, l = i % w.n_seq, i // w.n_seq
        d = w.directives[b]
        t0 = time.perf_counter()
        th = orope.inv_freq(64, 10000.0)
        p = osplice.plan(int(w.seq_lens[b]), int(d[0]), int(d[1]), int(d[2]), 0)
        r = kvsynth.rng(3, 9, b, l)
        pf = kvsynth.bf16_normal(r, (int(w.seq_lens[b]), 512))
        rp = kvsynth.bf16_normal(r, (int(w.seq_lens[b]), 64))
        spf = kvsynth.bf16_normal(r, (int(d[2]), 512))
        srp = kvsynth.bf16_normal(r, (int(d[2]), 64))
        t1 = time.perf_counter()
        osplice.splice_sequence(p, pf, rp, spf, srp, 1, 64, th)
        t2 = time.perf_counter()
        moved = p.moved_rows if p.delta != 0 else 0
        return moved / w.shape.n_layers, t2 - t1, t1 - t0


class SpliceLazy:
    """The batched-splice shape (64 sequences x 32768 slots, 64-row blocks)
    with each directive widened to block boundaries (s_start down, s_end and
    |R| up), done as block-table and pending-shift edits: no KV byte moves.
    Slots counted are the downstream slots re-indexed per step."""
    name = "lazy_splice"
    kernel = "lazy_kernel"
    dtype = "int32"
    data = "synthetic (seeded block tables, pending shifts and directives of the batched-splice draw)"

    def __init__(self):
        import kvsynth
        self.w = kvsynth.batched_splice()
        B = self.w.block_size
        d = self.w.directives
        s0 = d[:, 0] // B * B
        s1 = -(-d[:, 1] // B) * B
        rl = -(-d[:, 2] // B) * B
        # host inputs as a serving loop keeps them: int64 arrays, not Python lists
        self.dirs = np.stack([s0, s1, rl, np.zeros_like(s0)], axis=1).astype(np.int64)
        n = self.w.seq_lens.astype(np.int64)
        self.slots = int((n - s1).sum())
        nb_old = -(-n // B)
        nb_new = -(-(n + rl - (s1 - s0)) // B)
        # tables: both rows read up to the old count, written from s_start on;
        # stub ids read, freed ids written
        self.bytes = int((8 * nb_old + 8 * (np.maximum(nb_old, nb_new) - s0 // B) + 4 * (rl // B)
                          + 4 * ((s1 - s0) // B)).sum())
        self.launches = 1
        self.config = {"workload": "leyline_lazy_splices", "sequences": self.w.n_seq, "slots": self.w.capacity,
                       "block_size": B, "directives": "batched-splice draws widened to block boundaries",
                       "slots_per_step": self.slots, "kv_bytes_moved": 0,
                       "host_inputs": "directives [64, 4] and lengths [64] as int64 numpy arrays"}

    def setup(self):
        import torch
        import rope_rotation_splice_amd as rrs
        w = self.w
        self.bt = torch.from_numpy(w.block_tables.copy()).cuda()
        self.pend = torch.zeros_like(self.bt)
        n_stub = int((self.dirs[:, 2] // w.block_size).sum())
        self.stubs = torch.arange(w.n_blocks, w.n_blocks + n_stub, dtype=torch.int32, device="cuda")
        self.lens = w.seq_lens.astype(np.int64)
        self.rrs = rrs

    def step(self):
        # the same directives on the same lengths each step: same table work
        self.rrs.leyline_splice_lazy(self.bt, self.pend, self.w.block_size, self.lens, self.dirs, self.stubs)

    oracle_what = "sequence table edits of the step's directives (numpy)"

    def oracle_slabs(self):
        return self.w.n_seq

    def oracle_slab(self, i):
        from oracle import lazy as olazy
        w = self.w
        B = w.block_size
        pend = np.zeros(w.block_tables.shape[1], np.int64)
        stub = np.arange(64)
        d = self.dirs[i].tolist()
        t1 = time.perf_counter()
        n = 0
        while n == 0 or time.perf_counter() - t1 < 0.2:
            olazy.lazy_splice_tables(w.block_tables[i], pend, int(w.seq_lens[i]), d[0], d[1], d[2], B,
                                     stub[: d[2] // B])
            n += 1
        t2 = time.perf_counter()
        return n * (int(w.seq_lens[i]) - d[1]), t2 - t1, 0.0


class GatherLazy:
    """The registry-gather draw placed by reference: 32 entries kept in pool
    blocks (their lengths rounded down to whole 64-row blocks: rows past the
    last whole block would take the eager gather) packed at block-aligned
    targets in the draw's order.  Each step is one kv_relocate_gather_lazy
    call: table and pending-shift edits, no KV byte moves.  Slots counted are
    the entry rows placed per step."""
    name = "lazy_gather"
    kernel = "lazy_gather_kernel"
    dtype = "int32"
    data = "synthetic (the registry-gather draw of lengths, base positions and order; seeded block ids)"

    def __init__(self):
        import kvsynth
        self.w = kvsynth.registry_gather()
        w = self.w
        B = w.block_size
        nb = np.maximum(1, w.lens // B)
        order = np.argsort(w.p_target, kind="stable")
        tgt = np.zeros(len(nb), np.int64)
        k = 0
        for c in order:
            tgt[c] = k * B
            k += int(nb[c])
        self.nb, self.tgt, self.bt_stride = nb, tgt, int(k)
        self.slots = int((nb * B).sum())
        # per block: old id read, new id and shift written, entry id read, replaced id written
        self.bytes = int(20 * nb.sum())
        self.launches = 1
        self.config = {"workload": "irminsul_lazy_gather", "entries": len(nb), "block_size": B,
                       "entry_len": "U{256..2048} rounded down to whole blocks", "base_pos": "U{0..60000}",
                       "slots_per_step": self.slots, "kv_bytes_moved": 0}

    def setup(self):
        import torch
        import rope_rotation_splice_amd as rrs
        w, B = self.w, self.w.block_size
        r = np.random.default_rng(77)
        self.bt = torch.from_numpy(r.permutation(4 * self.bt_stride)[: self.bt_stride].astype(np.int32)
                                   .reshape(1, -1)).cuda()
        self.pend = torch.zeros_like(self.bt)
        ids = torch.arange(4 * self.bt_stride, 5 * self.bt_stride, dtype=torch.int32, device="cuda")
        self.ents, off = [], 0
        for c in range(len(self.nb)):
            n = int(self.nb[c])
            self.ents.append(rrs.LazyEntry(0, ids[off:off + n], n * B, int(w.base_pos[c]), int(self.tgt[c])))
            off += n
        self.batch = rrs.LazyBatch(self.ents)       # packed once, as a caller placing them repeatedly would
        self.rrs = rrs

    def step(self):
        self.rrs.kv_relocate_gather_lazy(self.bt, self.pend, self.w.block_size, self.batch)

    oracle_what = "table edits of the step's placements (numpy)"

    def oracle_slabs(self):
        return 1

    def oracle_slab(self, i):
        from oracle import lazy as olazy
        w, B = self.w, self.w.block_size
        bt = np.arange(self.bt_stride)
        pend = np.zeros(self.bt_stride, np.int64)
        pl, off = [], 0
        for c in range(len(self.nb)):
            n = int(self.nb[c])
            pl.append((np.arange(off, off + n), None, n * B, int(w.base_pos[c]), int(self.tgt[c])))
            off += n
        t1 = time.perf_counter()
        n = 0
        while n == 0 or time.perf_counter() - t1 < 0.2:
            olazy.lazy_gather_tables(bt, pend, B, pl)
            n += 1
        t2 = time.perf_counter()
        return n * self.slots, t2 - t1, 0.0


class Keys:
    """Registry keying of 64 token streams x 32768 tokens (vocab 131072): Gear
    CDC (threshold 2^56, chunks 64..2048 tokens), xxHash64 per chunk and per
    S1 128-token window.  Slots counted are tokens keyed."""
    name = "registry_keying"
    kernel = "gear_kernel + cut_kernel + fp_kernel"
    dtype = "u64"
    metric = "tokens keyed/sec (Gear CDC chunking + xxHash64 chunk and S1 fingerprints)"
    unit = "tokens/s"
    data = "synthetic (seeded token-id streams over shared documents, seeded 64-bit Gear table)"

    def __init__(self):
        import kvsynth
        self.w = kvsynth.registry_streams()
        n = self.w.tokens.size
        self.slots = n
        # tokens read by the hash pass and by the chunk and S1 fingerprint
        # passes, one Gear value per token, one candidate bit per token
        self.bytes = int(n * (4 * 3 + 8) + n / 8)
        self.launches = 1
        self.config = {"workload": "irminsul_registry_keying", "streams": self.w.tokens.shape[0],
                       "stream_len": self.w.tokens.shape[1], "vocab": len(self.w.gear), "threshold": "2^56",
                       "chunk_len": [self.w.min_len, self.w.max_len], "s1_window": self.w.s1_window,
                       "slots_per_step": n}

    def setup(self):
        import torch
        import rope_rotation_splice_amd as rrs
        w = self.w
        self.tok = torch.from_numpy(w.tokens.reshape(-1).copy()).cuda()
        self.gear = torch.from_numpy(w.gear.view(np.int64)).cuda()
        self.off = [int(x) for x in range(0, w.tokens.size + 1, w.tokens.shape[1])]
        self.rrs = rrs

    def step(self):
        w = self.w
        self.rrs.registry_chunk_keys(self.tok, self.off, self.gear, w.threshold, w.min_len, w.max_len, w.s1_window)

    oracle_what = "whole token streams of the same draw (pure Python)"

    def oracle_slabs(self):
        return self.w.tokens.shape[0]

    def oracle_slab(self, i):
        from oracle import keying as ok
        w = self.w
        t1 = time.perf_counter()
        ok.chunk_keys(w.tokens[i], w.gear, w.threshold, w.min_len, w.max_len, w.s1_window, w.seed)
        t2 = time.perf_counter()
        return w.tokens.shape[1], t2 - t1, 0.0


class GqaPatch:
    """Kamera GQA relocation with its rank-16 patch, fused into one gather:
    16 chunks x 1024 tokens, 32 layers, K and V of 8 x 128 bf16, delta ~
    U{-30000..30000}, RoPE base 500000, factors fp32 N(0, 0.01^2)."""
    name = "gqa_patch"
    kernel = "patch_dma_kernel<gather>"

    def __init__(self):
        import kvsynth
        self.w = kvsynth.gqa_patch()
        w = self.w
        L, n = w.shape.n_layers, len(w.deltas)
        width = w.shape.width
        self.slots = n * w.chunk_len
        factor_bytes = 2 * n * L * (w.chunk_len + width) * w.rank * 4
        self.bytes = self.slots * L * width * 2 * 2 * 2 + factor_bytes
        self.flops = 2 * 2 * n * L * w.chunk_len * width * w.rank
        self.launches = 1
        self.config = {"workload": "kamera_gqa_relocate_patch", "layers": L, "chunks": n, "chunk_len": w.chunk_len,
                       "kv_heads": w.shape.heads, "head_dim": w.shape.head_dim, "rope_base": w.shape.rope_base,
                       "delta": "U{-30000..30000}", "rank": w.rank, "factor_std": w.factor_std,
                       "slots_per_step": self.slots, "patch_gflop": self.flops / 1e9}

    def setup(self):
        import torch
        import kvsynth
        import rope_rotation_splice_amd as rrs
        w = self.w
        L, B, width, m = w.shape.n_layers, w.block_size, w.shape.width, w.rank
        self.K = torch.empty((L, w.n_blocks, B, width), dtype=torch.bfloat16, device="cuda")
        self.V = torch.empty_like(self.K)
        kvsynth.fill_normal_(self.K, 4, 1)
        kvsynth.fill_normal_(self.V, 4, 2)
        self.cache = rrs.KVCache.gqa(self.K, self.V, w.shape.heads, w.shape.head_dim, w.shape.rope_base)
        self.keep, self.ents, self.fk, self.fv = [], [], [], []
        for i in range(len(w.deltas)):
            ek = torch.empty((L, w.chunk_len, width), dtype=torch.bfloat16, device="cuda")
            ev = torch.empty_like(ek)
            kvsynth.fill_normal_(ek, 4, 3, i, 0)
            kvsynth.fill_normal_(ev, 4, 3, i, 1)
            self.ents.append(rrs.Rows(ev, ek, int(w.base_pos[i])))
            fac = []
            for j in range(4):
                shape = (L, w.chunk_len if j % 2 == 0 else width, m)
                t = torch.empty(shape, dtype=torch.float32, device="cuda")
                kvsynth.fill_normal_(t, 4, 4, i, j, std=w.factor_std)
                fac.append(t)
            self.fk.append(rrs.LowRank(fac[0], fac[1]))
            self.fv.append(rrs.LowRank(fac[2], fac[3]))
            self.keep += [ek, ev] + fac
        self.bt = torch.from_numpy(w.block_table).cuda()
        self.pt = w.p_target.tolist()
        self.rrs = rrs

    def step(self):
        self.rrs.kv_relocate_gather(self.cache, self.bt, self.ents, self.pt, self.fk, self.fv)

    oracle_what = "(chunk, layer) slabs, K rotated and patched, V patched (numpy fp64)"

    def oracle_slabs(self):
        return len(self.w.deltas) * self.w.shape.n_layers

    def oracle_slab(self, j):
        import kvsynth
        from oracle import patch as opatch, rope as orope, bf16 as ob
        w = self.w
        L = w.shape.n_layers
        i, l = j // L, j % L
        t0 = time.perf_counter()
        th = orope.inv_freq(w.shape.head_dim, w.shape.rope_base)
        r = kvsynth.rng(4, 9, i, l)
        k = ob.to_f64(kvsynth.bf16_normal(r, (w.chunk_len, w.shape.width)))
        v = ob.to_f64(kvsynth.bf16_normal(r, (w.chunk_len, w.shape.width)))
        U = kvsynth.f32_normal(r, (w.chunk_len, w.rank), w.factor_std)
        V = kvsynth.f32_normal(r, (w.shape.width, w.rank), w.factor_std)
        t1 = time.perf_counter()
        opatch.relocate_and_patch_keys(k, int(w.deltas[i]), w.shape.heads, w.shape.head_dim, th, U, V)
        opatch.patch_values(v, U, V)
        t2 = time.perf_counter()
        return w.chunk_len / L, t2 - t1, t1 - t0


class Decode:
    """Rotate-on-read absorbed-MLA decode: batch 32, 32768 cached tokens per
    sequence, 128 query heads (q_nope 512 + q_rope 64 bf16), paged 64-token
    blocks each carrying a pending shift ~ U{-1e5..1e5}, scale 1/sqrt(576).
    A slot is a key rotated on read."""
    name = "mla_decode"
    kernel = "mla_decode_kernel + combine"
    metric = "cached keys rotated on read and attended/sec (one decode step)"

    def __init__(self, zero_delta=False):
        import kvsynth
        self.w = kvsynth.rotate_on_read_decode()
        self.zero_delta = zero_delta
        w = self.w
        self.slots = w.batch * w.ctx
        cache = w.batch * w.ctx * 1152
        q = w.batch * w.heads * 576 * 2
        o = w.batch * w.heads * 512 * 2 + w.batch * w.heads * 4
        tables = 2 * w.block_tables.nbytes + w.seq_lens.nbytes
        self.bytes = cache + q + o + tables
        self.flops = 2 * w.batch * w.ctx * w.heads * (576 + 512)
        self.launches = 1
        if zero_delta:
            self.name = "mla_decode_zero_delta"
        self.config = {"workload": "mla_decode_rotate_on_read" + ("_zero_delta" if zero_delta else ""),
                       "batch": w.batch, "ctx": w.ctx, "heads": w.heads, "block_size": w.block_size,
                       "pending_delta": "0" if zero_delta else "U{-1e5..1e5} per block",
                       "q": "nope 512 + rope 64 bf16", "scale": "1/sqrt(576)", "keys_per_step": self.slots,
                       "gflop": self.flops / 1e9}

    def setup(self):
        import torch
        import kvsynth
        import rope_rotation_splice_amd as rrs
        w = self.w
        self.pool = torch.empty((1, w.n_blocks, w.block_size, 576), dtype=torch.bfloat16, device="cuda")
        kvsynth.fill_normal_(self.pool, 5, 1)
        self.qn = torch.empty((w.batch, w.heads, 512), dtype=torch.bfloat16, device="cuda")
        self.qr = torch.empty((w.batch, w.heads, 64), dtype=torch.bfloat16, device="cuda")
        kvsynth.fill_normal_(self.qn, 5, 2)
        kvsynth.fill_normal_(self.qr, 5, 3)
        self.cache = rrs.KVCache.mla(self.pool)
        self.bt = torch.from_numpy(w.block_tables).cuda()
        pend = np.zeros_like(w.pending_delta) if self.zero_delta else w.pending_delta
        self.pend = torch.from_numpy(pend).cuda()
        self.lens = torch.from_numpy(w.seq_lens).cuda()
        self.out = torch.empty((w.batch, w.heads, 512), dtype=torch.bfloat16, device="cuda")
        self.lse = torch.empty((w.batch, w.heads), dtype=torch.float32, device="cuda")
        self.rrs = rrs

    def step(self):
        w = self.w
        self.rrs.mla_decode_rotate_on_read(self.qn, self.qr, self.cache, 0, self.bt, self.pend, self.lens, w.scale,
                                           max_seq_len=w.ctx, out=self.out, lse=self.lse)

    oracle_what = "whole sequences (128 heads) attended on explicitly re-rotated keys (numpy fp64)"

    def oracle_slabs(self):
        return self.w.batch

    def oracle_slab(self, b):
        import kvsynth
        from oracle import decode as odec, rope as orope, bf16 as ob
        w = self.w
        t0 = time.perf_counter()
        th = orope.inv_freq(64, 10000.0)
        r = kvsynth.rng(5, 9, b)
        ckv = ob.to_f64(kvsynth.bf16_normal(r, (w.ctx, 512)))
        kr = ob.to_f64(kvsynth.bf16_normal(r, (w.ctx, 64)))
        qn = ob.to_f64(kvsynth.bf16_normal(r, (w.heads, 512)))
        qr = ob.to_f64(kvsynth.bf16_normal(r, (w.heads, 64)))
        d = odec.token_deltas(w.pending_delta[b], w.ctx, 64)
        t1 = time.perf_counter()
        odec.mla_decode(qn, qr, ckv, kr, d, w.scale, th)
        t2 = time.perf_counter()
        return w.ctx, t2 - t1, t1 - t0


class GqaDecode:
    """Rotate-on-read GQA decode: batch 32, 32768 cached tokens per sequence,
    32 query heads on 8 KV heads of 128 (K and V bf16, separate pools, RoPE
    base 500000), paged 64-token blocks each carrying a pending shift
    ~ U{-30000..30000}, scale 1/sqrt(128).  A slot is a key rotated on read
    (per KV head: 8 per token)."""
    name = "gqa_decode"
    kernel = "gqa_decode_kernel + combine"
    metric = "cached keys rotated on read and attended/sec (one decode step, per KV head)"

    def __init__(self):
        import kvsynth
        self.w = kvsynth.gqa_rotate_on_read_decode()
        w = self.w
        G, D = w.shape.heads, w.shape.head_dim
        self.slots = w.batch * w.ctx * G
        cache = w.batch * w.ctx * G * D * 2 * 2
        q = w.batch * w.q_heads * D * 2
        o = w.batch * w.q_heads * D * 2 + w.batch * w.q_heads * 4
        tables = 2 * w.block_tables.nbytes + w.seq_lens.nbytes
        self.bytes = cache + q + o + tables
        self.flops = 2 * w.batch * w.ctx * w.q_heads * 2 * D
        self.launches = 1
        self.config = {"workload": "gqa_decode_rotate_on_read", "batch": w.batch, "ctx": w.ctx,
                       "q_heads": w.q_heads, "kv_heads": G, "head_dim": D, "block_size": w.block_size,
                       "pending_delta": "U{-30000..30000} per block", "scale": "1/sqrt(128)",
                       "keys_per_step": self.slots, "gflop": self.flops / 1e9}

    def setup(self):
        import torch
        import kvsynth
        import rope_rotation_splice_amd as rrs
        w = self.w
        G, D = w.shape.heads, w.shape.head_dim
        self.kp = torch.empty((1, w.n_blocks, w.block_size, G * D), dtype=torch.bfloat16, device="cuda")
        self.vp = torch.empty_like(self.kp)
        self.q = torch.empty((w.batch, w.q_heads, D), dtype=torch.bfloat16, device="cuda")
        kvsynth.fill_normal_(self.kp, 7, 1)
        kvsynth.fill_normal_(self.vp, 7, 2)
        kvsynth.fill_normal_(self.q, 7, 3)
        self.cache = rrs.KVCache.gqa(self.kp, self.vp, G, D)
        self.bt = torch.from_numpy(w.block_tables).cuda()
        self.pend = torch.from_numpy(w.pending_delta).cuda()
        self.lens = torch.from_numpy(w.seq_lens).cuda()
        self.out = torch.empty((w.batch, w.q_heads, D), dtype=torch.bfloat16, device="cuda")
        self.lse = torch.empty((w.batch, w.q_heads), dtype=torch.float32, device="cuda")
        self.rrs = rrs

    def step(self):
        w = self.w
        self.rrs.gqa_decode_rotate_on_read(self.q, self.cache, 0, self.bt, self.pend, self.lens, w.scale,
                                           max_seq_len=w.ctx, out=self.out, lse=self.lse)

    oracle_what = "whole sequences attended on explicitly re-rotated keys (numpy fp64)"

    def oracle_slabs(self):
        return self.w.batch

    def oracle_slab(self, b):
        import kvsynth
        from oracle import decode as odec, rope as orope, bf16 as ob
        w = self.w
        G, D = w.shape.heads, w.shape.head_dim
        t0 = time.perf_counter()
        th = orope.inv_freq(D, 500000.0)
        r = kvsynth.rng(7, 9, b)
        k = ob.to_f64(kvsynth.bf16_normal(r, (w.ctx, G * D)))
        v = ob.to_f64(kvsynth.bf16_normal(r, (w.ctx, G * D)))
        q = ob.to_f64(kvsynth.bf16_normal(r, (w.q_heads, D)))
        d = odec.token_deltas(w.pending_delta[b], w.ctx, 64)
        t1 = time.perf_counter()
        odec.gqa_decode(q, k, v, d, w.scale, th, G)
        t2 = time.perf_counter()
        return w.ctx * G, t2 - t1, t1 - t0


class PatchForm:
    """Kamera patch formation on the GQA patch shape: 32 layers x 16 chunks x
    2 tensors = 1024 deficits of 1024 tokens x 1024 features (float32,
    energy in 32 feature directions), rank-16 factors by the randomized range
    finder (32-column sketch, two power steps: five products with each
    deficit).  With orders > 1 (the orbit patch) each deficit is the mean of
    that many order-specific deficits.  A unit is one deficit factored.

    For widths that are a multiple of 256 up to 1024 (this workload's), each
    power step Z = Delta^T (Delta X) is one pass over the deficit, so a step
    reads every deficit three times (two power steps and the final
    Y = Delta Z) for its five products; wider deficits take five passes."""
    kernel = "power_kernel + sketch_gemm + orth + eig"
    dtype = "f32"
    unit = "deficits/s"
    metric = "deficits factored/sec (rank-m patch factors by randomized SVD)"
    data = "synthetic (seeded deficits: Gaussian factors of 32 decaying directions plus dense noise)"

    def __init__(self, orders=1):
        import kvsynth
        self.w = kvsynth.patch_formation(orders=orders)
        w = self.w
        self.name = "patch_formation" if orders == 1 else "orbit_patch"
        per = w.rows * w.cols * 4
        self.slots = w.n
        # the mean of the orders (read them, write the mean), the passes over
        # each deficit, the 32-column sketches (one pass: Z written, then
        # read and written by each orthonormalization and the second power
        # step, read by the last product and the eigensolve: 9 Z-sized
        # transfers; Y written once and read once), the factors
        mean = w.n * per * (w.orders + 1) if w.orders > 1 else 0
        one_pass = w.cols % 256 == 0 and w.cols <= 1024
        passes = 3 if one_pass else 5
        zb, yb = w.n * w.cols * w.sketch * 4, w.n * w.rows * w.sketch * 4
        sk = 9 * zb + 2 * yb if one_pass else 9 * zb + 6 * yb
        self.bytes = mean + passes * w.n * per + sk + w.n * ((w.rows + w.cols) * w.rank + w.rank) * 4
        self.flops = 5 * 2 * w.n * w.rows * w.cols * w.sketch
        self.launches = 1
        self.config = {"workload": "kamera_patch_formation" if orders == 1 else "kamera_orbit_patch",
                       "deficits": w.n, "rows": w.rows, "cols": w.cols, "rank": w.rank, "sketch": w.sketch,
                       "power_steps": 2, "orders": w.orders, "energy_dirs": w.energy_dirs,
                       "deficits_per_step": w.n, "gflop": self.flops / 1e9}

    def setup(self):
        import torch
        import kvsynth
        import rope_rotation_splice_amd as rrs
        w = self.w
        shape = (w.n, w.orders, w.rows, w.cols) if w.orders > 1 else (w.n, w.rows, w.cols)
        self.d = torch.empty(shape, dtype=torch.float32, device="cuda")
        kvsynth.deficit_batch_(self.d, w.energy_dirs, w.decay, w.noise, *w.seed_keys, w.orders)
        self.omega = torch.from_numpy(w.omega).cuda()
        self.out = (torch.empty((w.n, w.rows, w.rank), dtype=torch.float32, device="cuda"),
                    torch.empty((w.n, w.cols, w.rank), dtype=torch.float32, device="cuda"),
                    torch.empty((w.n, w.rank), dtype=torch.float32, device="cuda"))
        self.rrs = rrs

    def step(self):
        self.rrs.kamera_patch_factors(self.d, self.w.rank, self.omega, out=self.out)

    oracle_what = "deficits factored by float64 SVD (numpy LAPACK)"

    def oracle_slabs(self):
        return self.w.n

    def oracle_slab(self, i):
        import torch
        import kvsynth
        from oracle import svd
        w = self.w
        t0 = time.perf_counter()
        shape = (1, w.orders, w.rows, w.cols) if w.orders > 1 else (1, w.rows, w.cols)
        d = torch.empty(shape, dtype=torch.float32)
        kvsynth.deficit_batch_(d, w.energy_dirs, w.decay, w.noise, *w.seed_keys, 9, i)
        x = d[0].double().numpy()
        t1 = time.perf_counter()
        svd.truncated_factors(svd.orbit_deficit(x) if w.orders > 1 else x, w.rank)
        t2 = time.perf_counter()
        return 1, t2 - t1, t1 - t0


class Copy:
    """A plain device-to-device copy (torch's copy kernel) of the registry
    gather's byte volume, or with ``batched`` of the batched splice's (64.5 GB
    read, 64.5 GB written): the practical read+write ceiling, and the
    known-size kernel that calibrates the HBM byte counters."""
    name = "copy"
    kernel = "torch copy_"

    def __init__(self, batched=False):
        if batched:
            w = SpliceBatched()
            self.nbytes, self.slots = w.bytes // 2 // 2 * 2, w.slots
        else:
            g = Gather()
            self.nbytes, self.slots = g.bytes // 2 // 2 * 2, g.slots
        self.bytes = 2 * self.nbytes
        self.launches = 1
        self.config = {"workload": "device_copy_batched_splice_volume" if batched else "device_copy",
                       "bytes_read": self.nbytes, "bytes_written": self.nbytes}

    def setup(self):
        import torch
        self.a = torch.empty(self.nbytes // 2, dtype=torch.bfloat16, device="cuda").normal_()
        self.b = torch.empty_like(self.a)

    def step(self):
        self.b.copy_(self.a)

    oracle_what = None


WORKLOADS = {"gather": Gather, "splice": Splice, "splice_batched": SpliceBatched, "splice_lazy": SpliceLazy,
             "gather_lazy": GatherLazy,
             "gqa_patch": GqaPatch, "keys": Keys,
             "decode": Decode, "decode_zero_delta": lambda: Decode(zero_delta=True), "gqa_decode": GqaDecode,
             "patch_form": PatchForm, "orbit_patch": lambda: PatchForm(orders=4), "copy": Copy,
             "copy_batched": lambda: Copy(batched=True)}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="splice_batched", choices=sorted(WORKLOADS))
    ap.add_argument("--cpu-budget", type=float, default=4.0,
                    help="seconds of oracle time per worker process for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (relocation shards with no "
              "exchange; see the sharding paragraph of the design notes). Run with --gpus 1.", file=sys.stderr)
        return 2

    wl = WORKLOADS[args.workload]()
    unit = getattr(wl, "unit", "keys/s" if isinstance(wl, (Decode, GqaDecode)) else "slots/s")
    # the CPU oracle runs before the GPU is touched
    cpu = None
    if not args.no_cpu_baseline and wl.oracle_what:
        cpu = oracle_baseline(args.workload, args.cpu_budget, unit, wl.oracle_what)

    import torch
    torch.cuda.set_device(0)
    wl.setup()
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        wl.step()
    torch.cuda.synchronize()
    import rope_rotation_splice_amd as rrs
    if rrs.device_errors():
        raise SystemExit("device error flags set during warmup")

    stream = torch.cuda.current_stream()          # the library launches on this stream
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        wl.step()
    ev1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall = t1 - t0
    gpu_s = ev0.elapsed_time(ev1) / 1e3
    if rrs.device_errors():
        raise SystemExit("device error flags set during the timed steps")

    # Spread of single steps, outside the timed region: up to 20 more steps,
    # each between its own events (host enqueue gaps included).
    per_us = []
    for _ in range(min(20, args.steps)):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        wl.step()
        e1.record(stream)
        e1.synchronize()
        per_us.append(e0.elapsed_time(e1) * 1e3)
    if rrs.device_errors():
        raise SystemExit("device error flags set during the per-step timing")

    launches = args.steps * wl.launches
    kernel_s = gpu_s / launches
    bytes_per_launch = wl.bytes / wl.launches
    achieved = bytes_per_launch / kernel_s / 1e9
    traffic = stored_traffic(wl.kernel, wl.name)
    extra = {}
    if getattr(wl, "flops", None):
        dt, peak = ("bf16", 2500.0) if isinstance(wl, (Decode, GqaDecode)) else ("fp32", 157.3)
        extra["matrix_core"] = {"dtype": dt, "achieved_TFLOPs": wl.flops * args.steps / gpu_s / 1e12,
                                "peak_TFLOPs": peak, "frac": wl.flops * args.steps / gpu_s / 1e12 / peak}
    out = {
        "metric": getattr(wl, "metric", METRIC),
        "value": wl.slots * args.steps / wall,
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": getattr(wl, "dtype", "bf16"),
        "data": getattr(wl, "data", "synthetic (seeded N(0,1) bf16 cache rows, integer draws as stated in config)"),
        "config": wl.config,
        "hbm_GBps_per_step": wl.bytes * args.steps / wall / 1e9,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": wl.kernel, "algorithmic_bytes_per_launch": bytes_per_launch,
                     "avg_launch_us": kernel_s * 1e6},
        "cpu_baseline": cpu,
    }
    if per_us:
        out["step_us"] = {"median": float(np.median(per_us)), "min": float(min(per_us)), "n": len(per_us)}
    out.update(extra)
    if hasattr(wl, "extra"):
        out.update(wl.extra())
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
