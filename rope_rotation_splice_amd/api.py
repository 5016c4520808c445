"""Python entry points over the C ABI (torch tensors in, ctypes out).

Argument marshalling only: every step of the relocation runs in the HIP
library.  Tensors supply device memory, torch's current stream supplies the
HIP stream.  Calls are asynchronous like any torch op; keep the tensors alive
until the stream has run them.
"""

import ctypes
from dataclasses import dataclass

import numpy as np
import torch

from . import _abi
from ._abi import (kvr_cdc_params, KVR_AMORTIZE, KVR_BF16, KVR_F32, KVR_FORGET, KVR_FORGET_NEEDS_PREFILL,  # noqa: F401
                   KVR_E_WORKSPACE, KVR_OK, kvr_cache, kvr_directive, kvr_lowrank, kvr_part, kvr_rows)


class KVRError(RuntimeError):
    def __init__(self, fn, status):
        lib = _abi.load()
        msg = lib.kvr_status_str(status).decode()
        if status == -5:
            msg += f" (hipError {lib.kvr_last_hip_error()})"
        super().__init__(f"{fn}: {msg} [status {status}]")
        self.status = status


def _check(fn, st):
    if st < 0:
        raise KVRError(fn, st)
    return st


_DT = {torch.bfloat16: KVR_BF16, torch.float32: KVR_F32}


# Argument checks made before any library call.  The library sees only raw
# addresses, so a host tensor, a tensor on another GPU, a wrong dtype or a
# short table would make its kernels read or write the wrong memory; these
# raise ValueError instead.  Structure (dtype, shape) is checked before the
# device, so that the checks can be exercised without a GPU.

def _need(cond, msg):
    """Raise ValueError(msg) unless cond; msg may be a callable that builds
    the message, so that passing checks format nothing."""
    if not cond:
        raise ValueError(msg() if callable(msg) else msg)


def _on(t, device, name):
    _need(t.is_cuda, lambda: f"{name} must be a CUDA tensor")
    _need(t.device == device, lambda: f"{name} is on {t.device}, expected {device}")


def _i32(t, name, dims=None, contiguous=True):
    _need(isinstance(t, torch.Tensor), lambda: f"{name} must be a torch tensor")
    _need(t.dtype == torch.int32, lambda: f"{name} must be int32, got {t.dtype}")
    if dims is not None:
        _need(t.dim() == dims, lambda: f"{name} must have {dims} dimensions")
    if contiguous:
        _need(t.is_contiguous(), lambda: f"{name} must be contiguous")


def _tensor(t, name, dtype, shape):
    """dtype, exact shape (None entries free) and contiguity."""
    if isinstance(t, torch.Tensor) and t.dtype == dtype:
        sh = t.shape
        if len(sh) == len(shape) and all(s is None or a == s for a, s in zip(sh, shape)) and t.is_contiguous():
            return
    _need(isinstance(t, torch.Tensor), lambda: f"{name} must be a torch tensor")
    _need(t.dtype == dtype, lambda: f"{name} must be {dtype}, got {t.dtype}")
    _need(t.dim() == len(shape) and all(s is None or int(a) == s for a, s in zip(t.shape, shape)),
          lambda: f"{name} has shape {tuple(t.shape)}, expected {tuple('*' if s is None else s for s in shape)}")
    _need(t.is_contiguous(), lambda: f"{name} must be contiguous")


# The current device's current stream as a raw handle.  torch's private
# accessor skips building a Stream object (about 3 us per call); the public
# route is kept for builds without it.
_raw_stream_of = getattr(torch._C, "_cuda_getCurrentRawStream", None)
_get_device = getattr(torch._C, "_cuda_getDevice", None)


def _raw_stream():
    if _raw_stream_of is not None and _get_device is not None:
        return _raw_stream_of(_get_device())
    return torch.cuda.current_stream().cuda_stream


def _stream_handle():
    return ctypes.c_void_p(_raw_stream())


def _part(t):
    """kvr_part of a [layers, blocks, rows, width] view with a unit last stride."""
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError("cache parts must be [layers, blocks, rows, width] views with unit last stride")
    return kvr_part(t.data_ptr(), t.stride(0), t.stride(1), t.stride(2))


class KVCache:
    """A paged KV cache: ``pf`` (position-free part) and ``rope`` (rotary part)
    as [layers, blocks, block_size, width] tensor views."""

    def __init__(self, pf, rope, rope_heads, rope_dim, rope_base, inv_freq=None):
        if pf.shape[:3] != rope.shape[:3]:
            raise ValueError("pf and rope views must share layers, blocks and rows")
        if rope.shape[3] != rope_heads * rope_dim:
            raise ValueError("rope width must be rope_heads * rope_dim")
        if pf.dtype not in _DT or rope.dtype not in _DT:
            raise ValueError("cache parts must be bfloat16 or float32")
        if pf.device != rope.device:
            raise ValueError("pf and rope views must live on one device")
        self.pf, self.rope = pf, rope
        self.device = pf.device
        self.pf_width, self.rope_width = int(pf.shape[3]), int(rope.shape[3])
        self.pf_dtype, self.rope_dtype = pf.dtype, rope.dtype
        self.n_layers, self.n_blocks, self.block_size = (int(x) for x in pf.shape[:3])
        self.rope_heads, self.rope_dim, self.rope_base = rope_heads, rope_dim, float(rope_base)
        self._inv = None
        if inv_freq is not None:
            self._inv = (ctypes.c_double * (rope_dim // 2))(*[float(x) for x in inv_freq])
        self.c = kvr_cache(self.n_layers, self.block_size, self.n_blocks, int(pf.shape[3]), _DT[pf.dtype],
                           rope_heads, rope_dim, _DT[rope.dtype], self.rope_base,
                           ctypes.cast(self._inv, ctypes.POINTER(ctypes.c_double)) if self._inv else None,
                           _part(pf), _part(rope))

    @classmethod
    def mla(cls, pool, pf_width=512, rope_dim=64, rope_base=10000.0):
        """MLA pool [layers, blocks, block_size, 576]: row = [cKV | k_rope]."""
        return cls(pool[..., :pf_width], pool[..., pf_width:], 1, rope_dim, rope_base)

    @classmethod
    def gqa(cls, k, v, heads, head_dim, rope_base=500000.0):
        """GQA pools K, V [layers, blocks, block_size, heads*head_dim]."""
        return cls(v, k, heads, head_dim, rope_base)


@dataclass
class Rows:
    """Token rows outside the pool for every layer: pf [layers, len, pf_w],
    rope [layers, len, rope_w] (unit last stride).  A registry entry
    (cKV, k_r, base_pos) or a splice stub."""
    pf: torch.Tensor
    rope: torch.Tensor
    base_pos: int = 0

    def check(self, cache, name="rows", device=True):
        """Layers, widths, dtypes and (with ``device``) device must match the cache's parts."""
        pf, rp = self.pf, self.rope
        ps, rs = pf.shape, rp.shape
        if (len(ps) == 3 and len(rs) == 3 and ps[0] == cache.n_layers and rs[0] == cache.n_layers and ps[1] == rs[1]
                and ps[2] == cache.pf_width and rs[2] == cache.rope_width
                and pf.dtype == cache.pf_dtype and rp.dtype == cache.rope_dtype):
            if device and ps[1] and not (pf.is_cuda and rp.is_cuda and pf.device == cache.device
                                         and rp.device == cache.device):
                _on(pf, cache.device, f"{name}.pf")
                _on(rp, cache.device, f"{name}.rope")
            return
        _need(pf.dim() == 3 and rp.dim() == 3, lambda: f"{name}: pf and rope must be [layers, len, width]")
        _need(int(pf.shape[0]) == cache.n_layers and int(rp.shape[0]) == cache.n_layers,
              lambda: f"{name}: {int(pf.shape[0])} layers, the cache has {cache.n_layers}")
        _need(int(pf.shape[1]) == int(rp.shape[1]), lambda: f"{name}: pf and rope lengths differ")
        _need(int(pf.shape[2]) == int(cache.pf.shape[3]) and int(rp.shape[2]) == int(cache.rope.shape[3]),
              lambda: f"{name}: widths {int(pf.shape[2])}/{int(rp.shape[2])} differ from the cache's")
        _need(pf.dtype == cache.pf.dtype and rp.dtype == cache.rope.dtype, lambda: f"{name}: dtypes differ from the cache's")
        if device and int(pf.shape[1]):
            _on(pf, cache.device, f"{name}.pf")
            _on(rp, cache.device, f"{name}.rope")

    def c(self):
        if self.pf.shape[1] == 0:
            return kvr_rows()             # no rows: nothing to copy
        if self.pf.stride(-1) != 1 or self.rope.stride(-1) != 1:
            raise ValueError("rows need a unit last stride")
        return kvr_rows(self.pf.data_ptr(), self.pf.stride(0), self.pf.stride(1),
                        self.rope.data_ptr(), self.rope.stride(0), self.rope.stride(1),
                        int(self.pf.shape[1]), int(self.base_pos))


@dataclass
class LowRank:
    """fp32 factors for every layer: U [layers, len, rank], V [layers, width, rank]."""
    U: torch.Tensor
    V: torch.Tensor

    def check(self, device, layers, rows, width, name="factors", on_device=True):
        U, V = self.U, self.V
        if isinstance(U, torch.Tensor) and isinstance(V, torch.Tensor):
            us, vs = U.shape, V.shape
            if (len(us) == 3 and len(vs) == 3 and us[0] == layers and us[1] == rows and vs[0] == layers
                    and vs[1] == width and vs[2] == us[2] and U.dtype == torch.float32 and V.dtype == torch.float32
                    and U.is_contiguous() and V.is_contiguous()):
                if on_device and us[0] * us[1] * us[2]:
                    _on(U, device, f"{name}.U")
                    _on(V, device, f"{name}.V")
                return
        _need(U.dim() == 3 and V.dim() == 3, lambda: f"{name}: U and V must be [layers, n, rank]")
        r = int(U.shape[2])
        _tensor(U, f"{name}.U", torch.float32, (layers, rows, r))
        _tensor(V, f"{name}.V", torch.float32, (layers, width, r))
        if on_device and U.numel():
            _on(U, device, f"{name}.U")
            _on(V, device, f"{name}.V")

    def c(self):
        r = int(self.U.shape[-1])
        if self.U.numel() == 0:
            return kvr_lowrank()          # no rows to patch
        if not (self.U.is_contiguous() and self.V.is_contiguous()) or self.U.dtype != torch.float32:
            raise ValueError("factors must be contiguous float32")
        return kvr_lowrank(self.U.data_ptr(), self.U.stride(0), self.V.data_ptr(), self.V.stride(0), r, 0)


_workspaces = {}


def _workspace(nbytes, device, kind, raw_stream=None):
    """A workspace per (kind, device, stream).  Kinds never share memory: the
    splice's must stay zero-filled between calls (each call leaves it so),
    the decode's holds split partials."""
    raw_stream = raw_stream if raw_stream is not None else _raw_stream()
    key = (kind, device.index if device.index is not None else torch.cuda.current_device(), raw_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


# numpy mirror of kvr_directive (three int64, mode, reserved), filled in one
# vectorized pass; the ctypes pointer keeps the array alive
_DIR_DT = np.dtype([("s_start", "<i8"), ("s_end", "<i8"), ("r_len", "<i8"), ("mode", "<i4"), ("reserved", "<i4")])
assert _DIR_DT.itemsize == ctypes.sizeof(kvr_directive)
# numpy mirror of kvr_lazy_entry (seq, padding, two device pointers, three int64)
_LAZY_DT = np.dtype([("seq", "<i4"), ("pad", "<i4"), ("d_blocks", "<u8"), ("d_pend", "<u8"), ("len", "<i8"),
                     ("base_pos", "<i8"), ("p_target", "<i8")])
assert _LAZY_DT.itemsize == ctypes.sizeof(_abi.kvr_lazy_entry)


class _HostArray:
    """A host array handed to the library as a typed pointer: a ctypes array
    (cheapest for a few items) or a numpy array (cheapest for many; holding
    this object keeps it alive for the call, since ctypes.cast keeps no
    reference and ndarray.ctypes.data_as is slow)."""
    __slots__ = ("a", "p")

    def __init__(self, a, ctype=None):
        self.a = a
        self.p = a if ctype is None else ctypes.cast(a.ctypes.data, ctypes.POINTER(ctype))

    def values(self, n):
        return np.array(self.a[:n], dtype=np.int64)


_FEW = 8      # below this many items plain ctypes arrays are cheaper than numpy


def _directives(directives):
    """(host array of kvr_directive, count); pass ``.p`` to the library."""
    n = len(directives)
    if n <= _FEW:
        return _HostArray((kvr_directive * max(1, n))(*[kvr_directive(int(s), int(e), int(r), int(m), 0)
                                                        for s, e, r, m in directives])), n
    d = np.asarray(directives, dtype=np.int64).reshape(-1, 4)
    arr = np.zeros(len(d), dtype=_DIR_DT)
    arr["s_start"], arr["s_end"], arr["r_len"], arr["mode"] = d[:, 0], d[:, 1], d[:, 2], d[:, 3]
    return _HostArray(arr, kvr_directive), len(d)


def _i64(values, n):
    """A host int64 array of at least one element (the first n from values)."""
    if n <= _FEW:
        return _HostArray((ctypes.c_int64 * max(1, n))(*[int(values[i]) for i in range(n)]))
    a = np.asarray(values, dtype=np.int64).reshape(-1)[:n].copy()
    return _HostArray(a, ctypes.c_int64)


def splice_workspace_bytes(cache, seq_lens, directives):
    lib = _abi.load()
    dirs, n = _directives(directives)
    lens = _i64(seq_lens, n)
    return int(lib.kvr_splice_workspace_bytes(ctypes.byref(cache.c), n, lens.p, dirs.p))


def _splice_args(cache, block_tables, seq_lens, directives, stubs):
    """Checked host arrays for leyline_splice and leyline_splice_noalloc:
    (directives, n, lengths, new-length output, stub array)."""
    dirs, n = _directives(directives)
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.stride(1) != 1:
        raise ValueError("block_tables must be an int32 [n_seq, blocks] tensor with unit last stride")
    _need(int(block_tables.shape[0]) >= n, "block_tables needs a row per directive")
    _need(len(seq_lens) == n, "seq_lens needs one length per directive")
    if stubs is not None:
        _need(len(stubs) == n, "stubs needs one entry (Rows or None) per directive")
        for i, s in enumerate(stubs):
            if s is not None:
                s.check(cache, f"stubs[{i}]", device=False)
    _on(block_tables, cache.device, "block_tables")
    lens, out = _i64(seq_lens, n), _i64(np.zeros(n, np.int64), n)
    stub_arr = None
    if stubs is not None:
        stub_arr = (kvr_rows * max(1, n))()
        dev = cache.device
        for i, s in enumerate(stubs):
            if s is not None:
                # structure passed above; now the device
                if s.pf.shape[1] and not (s.pf.is_cuda and s.rope.is_cuda and s.pf.device == dev
                                          and s.rope.device == dev):
                    _on(s.pf, dev, f"stubs[{i}].pf")
                    _on(s.rope, dev, f"stubs[{i}].rope")
                stub_arr[i] = s.c()
    return dirs, n, lens, out, stub_arr


def leyline_splice(cache, block_tables, seq_lens, directives, stubs=None, workspace=None):
    """In-place AMORTIZE/FORGET splices, one directive (s_start, s_end, r_len, mode) per sequence.

    block_tables: int32 device tensor [n_seq, blocks_per_seq].  stubs: list of
    Rows (or None per sequence) holding the prefilled replacement rows.
    Returns (new_lens int64 array, status) -- status 1 means a FORGET was seen.
    """
    lib = _abi.load()
    dirs, n, lens, out, stub_arr = _splice_args(cache, block_tables, seq_lens, directives, stubs)
    stream = _raw_stream()
    handle = ctypes.c_void_p(stream)

    def call(ws):
        return lib.leyline_splice(ctypes.byref(cache.c), block_tables.data_ptr(), int(block_tables.stride(0)), n,
                                  lens.p, dirs.p, stub_arr, out.p, ws.data_ptr(), ws.numel() * ws.element_size(),
                                  handle)

    if workspace is not None:
        st = call(workspace)
    else:
        # The cached workspace usually fits; a call it does not fit fails
        # validation before anything is enqueued, and is repeated once with
        # a workspace of the queried size.
        st = call(_workspace(0, cache.pf.device, "splice", stream))
        if st == KVR_E_WORKSPACE:
            need = lib.kvr_splice_workspace_bytes(ctypes.byref(cache.c), n, lens.p, dirs.p)
            st = call(_workspace(need, cache.pf.device, "splice", stream))
    _check("leyline_splice", st)
    return out.values(n), st


def leyline_splice_noalloc(cache, block_tables, seq_lens, directives, stubs=None):
    """leyline_splice without any workspace or allocation: the library's own
    per-GPU device scratch holds the ordering state (see
    kvr_noalloc_scratch_bytes).  Calls that overlap on one GPU race.
    Returns (new_lens int64 array, status)."""
    lib = _abi.load()
    dirs, n, lens, out, stub_arr = _splice_args(cache, block_tables, seq_lens, directives, stubs)
    st = lib.leyline_splice_noalloc(ctypes.byref(cache.c), block_tables.data_ptr(), int(block_tables.stride(0)), n,
                                    lens.p, dirs.p, stub_arr, out.p, _stream_handle())
    _check("leyline_splice_noalloc", st)
    return out.values(n), st


def leyline_splice_lazy(block_tables, pending_delta, block_size, seq_lens, directives, stub_blocks=None):
    """Block-aligned AMORTIZE splices done as edits of the block table and of
    the per-block pending shifts (no KV bytes move); decode with
    mla_decode_rotate_on_read applies the composed shift on read.

    block_tables, pending_delta: int32 device tensors [n_seq, bt_stride],
    edited in place.  stub_blocks: int32 device tensor with the r_len /
    block_size prefilled block ids of every sequence, concatenated in order.
    Returns (new_lens int64 array, freed int32 device tensor, status).
    """
    lib = _abi.load()
    dirs, n = _directives(directives)
    for t in (block_tables, pending_delta):
        if t.dtype != torch.int32 or t.dim() != 2 or t.stride(1) != 1:
            raise ValueError("block_tables and pending_delta must be int32 [n_seq, blocks] with unit last stride")
    if pending_delta.shape != block_tables.shape or pending_delta.stride(0) != block_tables.stride(0):
        raise ValueError("pending_delta must match block_tables in shape and row stride")
    _need(int(block_tables.shape[0]) >= n, "block_tables needs a row per directive")
    _need(len(seq_lens) == n, "seq_lens needs one length per directive")
    _on(block_tables, block_tables.device, "block_tables")
    _on(pending_delta, block_tables.device, "pending_delta")
    if n > _FEW:
        da = dirs.a
        n_free = int(((da["s_end"] - da["s_start"]) // block_size)[da["mode"] == 0].sum())
    else:
        n_free = sum(int((d[1] - d[0]) // block_size) for d in directives if int(d[3]) == KVR_AMORTIZE)
    if stub_blocks is not None and (stub_blocks.dtype != torch.int32 or not stub_blocks.is_contiguous()):
        raise ValueError("stub_blocks must be a contiguous int32 tensor")
    if stub_blocks is not None and stub_blocks.numel():
        _on(stub_blocks, block_tables.device, "stub_blocks")
    freed = torch.empty(max(1, n_free), dtype=torch.int32, device=block_tables.device)
    lens, out = _i64(seq_lens, n), _i64(np.zeros(n, np.int64), n)
    st = lib.leyline_splice_lazy(int(block_size), block_tables.data_ptr(), pending_delta.data_ptr(),
                                 int(block_tables.stride(0)), n, lens.p, dirs.p,
                                 stub_blocks.data_ptr() if stub_blocks is not None and stub_blocks.numel() else None,
                                 freed.data_ptr() if n_free else None, out.p, _stream_handle())
    _check("leyline_splice_lazy", st)
    return out.values(n), freed[:n_free], st


class LazyEntry:
    """A registry entry kept in pool blocks (row 0 at the start of blocks[0]),
    placed by reference at ``p_target`` of sequence ``seq``.  blocks: int32
    device tensor [ceil(len / block_size)]; pend: the shifts those blocks
    already owe (int32 device tensor of the same length) or None.  The
    tensors are checked and their addresses taken once, here: an entry is
    immutable, and its tensors must not be resized while it is in use."""
    __slots__ = ("_seq", "_blocks", "_pend", "_len", "_base", "_target", "_row", "_n_blocks", "_n_pend",
                 "_device")

    def __init__(self, seq, blocks, length, base_pos, p_target, pend=None):
        for t in (blocks, pend):
            if t is not None and (t.dtype != torch.int32 or not t.is_contiguous()):
                raise ValueError("entry blocks and pend must be contiguous int32 tensors")
        if blocks is not None and pend is not None and blocks.device != pend.device:
            raise ValueError("entry blocks and pend must live on one device")
        self._device = blocks.device if blocks is not None else None
        self._seq, self._blocks, self._pend, self._len = int(seq), blocks, pend, int(length)
        self._base, self._target = int(base_pos), int(p_target)
        self._n_blocks = blocks.numel() if blocks is not None else 0
        self._n_pend = pend.numel() if pend is not None else None
        self._row = (self._seq, 0, blocks.data_ptr() if self._n_blocks else 0,
                     pend.data_ptr() if pend is not None and self._n_pend else 0,
                     self._len, self._base, self._target)

    seq = property(lambda self: self._seq)
    blocks = property(lambda self: self._blocks)
    pend = property(lambda self: self._pend)
    len = property(lambda self: self._len)
    base_pos = property(lambda self: self._base)
    p_target = property(lambda self: self._target)


class LazyBatch:
    """LazyEntry objects packed once into the host array the library reads,
    for callers that place the same entries repeatedly (entries are
    immutable, and the batch keeps its own tuple of them)."""
    __slots__ = ("entries", "_host", "_totals")

    def __init__(self, entries):
        self.entries = tuple(entries)
        arr = np.array([e._row for e in self.entries] or [(0, 0, 0, 0, 0, 0, 0)], dtype=_LAZY_DT)
        self._host = _HostArray(arr, _abi.kvr_lazy_entry)
        self._totals = {}          # block size -> checked block count

    def __len__(self):
        return len(self.entries)


def kv_relocate_gather_lazy(block_tables, pending_delta, block_size, entries):
    """Registry entries placed at block-aligned targets as edits of the block
    table and of the per-block pending shifts (no KV bytes move); decode with
    mla_decode_rotate_on_read applies the shift on read.

    block_tables, pending_delta: int32 device tensors [n_seq, bt_stride],
    edited in place.  entries: a list of LazyEntry, or a LazyBatch of them.
    Returns (replaced int32 device tensor: the ids each entry's logical
    blocks held before, entry after entry; status).
    """
    lib = _abi.load()
    for t in (block_tables, pending_delta):
        if t.dtype != torch.int32 or t.dim() != 2 or t.stride(1) != 1:
            raise ValueError("block_tables and pending_delta must be int32 [n_seq, blocks] with unit last stride")
    if pending_delta.shape != block_tables.shape or pending_delta.stride(0) != block_tables.stride(0):
        raise ValueError("pending_delta must match block_tables in shape and row stride")
    _on(block_tables, block_tables.device, "block_tables")
    _on(pending_delta, block_tables.device, "pending_delta")
    batch = entries if isinstance(entries, LazyBatch) else None
    items = batch.entries if batch is not None else entries
    n = len(items)
    B = int(block_size)
    key = (B, block_tables.device, int(block_tables.shape[0]))
    total = batch._totals.get(key) if batch is not None else None
    if total is None:
        total = 0
        for e in items:
            nb = -(-e._len // B) if e._len > 0 else 0
            if e._n_blocks < nb or (e._n_pend is not None and e._n_pend < nb):
                raise ValueError("entry blocks and pend need ceil(len / block_size) ids")
            _need(0 <= e._seq < int(block_tables.shape[0]), "entry sequence outside the block tables")
            if nb:
                _need(e._device == block_tables.device, "entry blocks must live on the block tables' device")
            total += nb
        if batch is not None:
            batch._totals[key] = total
    if batch is not None:
        ents = batch._host
    else:
        arr = np.array([e._row for e in items] or [(0, 0, 0, 0, 0, 0, 0)], dtype=_LAZY_DT)
        ents = _HostArray(arr, _abi.kvr_lazy_entry)
    replaced = torch.empty(max(1, total), dtype=torch.int32, device=block_tables.device)
    st = lib.kv_relocate_gather_lazy(int(block_size), block_tables.data_ptr(), pending_delta.data_ptr(),
                                     int(block_tables.stride(0)), int(block_tables.shape[0]), ents.p, n,
                                     replaced.data_ptr() if total else None, _stream_handle())
    _check("kv_relocate_gather_lazy", st)
    return replaced[:total], st


def registry_chunk_keys(tokens, offsets, gear, threshold, min_len, max_len, s1_window, seed=0,
                        with_hash=False, with_s1=True):
    """Content-defined chunking of token streams with a Gear rolling hash and
    xxHash64 fingerprints, plus S1 fixed windows per chunk.

    tokens: int32 device tensor (streams concatenated); offsets: host list of
    n_streams + 1 token offsets; gear: device tensor of 64-bit values per token
    id (int64 or uint64 storage).  Returns a dict with chunk_end [n, cap],
    n_chunks [n], chunk_fp [n, cap] (int64 storage of uint64), s1_fp
    [n, cap, slots] and, on request, hash [total].  Rows of chunk_end,
    chunk_fp and s1_fp past n_chunks[s] are left unwritten (unspecified).
    """
    lib = _abi.load()
    if tokens.dtype != torch.int32 or not tokens.is_contiguous():
        raise ValueError("tokens must be a contiguous int32 tensor")
    if gear.element_size() != 8 or not gear.is_contiguous():
        raise ValueError("gear must be a contiguous tensor of 64-bit values")
    _need(len(offsets) >= 1, "offsets needs n_streams + 1 entries")
    _need(int(tokens.numel()) >= int(offsets[-1]), "tokens is shorter than the last offset")
    _on(tokens, tokens.device, "tokens")
    _on(gear, tokens.device, "gear")
    off = [int(x) for x in offsets]
    n = len(off) - 1
    lens = [off[i + 1] - off[i] for i in range(n)]
    cap = max([1] + [-(-ln // int(min_len)) for ln in lens])
    slots = -(-int(max_len) // int(s1_window))
    dev = tokens.device
    out = {"chunk_end": torch.empty((max(n, 1), cap), dtype=torch.int32, device=dev)[:n],
           "n_chunks": torch.empty(max(n, 1), dtype=torch.int32, device=dev)[:n],
           "chunk_fp": torch.empty((max(n, 1), cap), dtype=torch.int64, device=dev)[:n]}
    out["s1_fp"] = torch.empty((max(n, 1), cap, slots), dtype=torch.int64, device=dev)[:n] if with_s1 else None
    out["hash"] = torch.zeros(max(1, off[-1] if n else 1), dtype=torch.int64, device=dev) if with_hash else None
    p = kvr_cdc_params(int(threshold), int(min_len), int(max_len), int(s1_window), 0, int(seed))
    offs = (ctypes.c_int64 * max(1, n + 1))(*off)
    need = lib.kvr_keys_workspace_bytes(off[-1] - off[0] if n else 0)
    ws = _workspace(need, dev, "keys")
    ptr = lambda t: t.data_ptr() if t is not None else None
    st = lib.registry_chunk_keys(tokens.data_ptr(), offs, n, gear.data_ptr(), int(gear.numel()), ctypes.byref(p),
                                 ptr(out["hash"]), ptr(out["chunk_end"]), cap, ptr(out["n_chunks"]),
                                 ptr(out["chunk_fp"]), ptr(out["s1_fp"]), ws.data_ptr(), ws.numel(), _stream_handle())
    _check("registry_chunk_keys", st)
    return out


def kv_relocate_gather(cache, block_table, entries, p_targets, patch_rope=None, patch_pf=None):
    """Gather registry entries (list of Rows) into one paged destination
    sequence at logical slots p_targets[i] + t; optional rank-m patches
    (lists of LowRank or None)."""
    lib = _abi.load()
    n = len(entries)
    if block_table.dtype != torch.int32 or block_table.dim() != 1 or block_table.stride(0) != 1:
        raise ValueError("block_table must be a contiguous int32 [blocks] tensor")
    _need(len(p_targets) == n, "p_targets needs one target per entry")
    patches = ((patch_rope, int(cache.rope.shape[3]), "patch_rope"), (patch_pf, int(cache.pf.shape[3]), "patch_pf"))
    for on_device in (False, True):
        for i, e in enumerate(entries):
            e.check(cache, f"entries[{i}]", device=on_device)
        for lst, width, name in patches:
            if lst is None:
                continue
            _need(len(lst) == n, lambda: f"{name} needs one entry (LowRank or None) per registry entry")
            for i, f in enumerate(lst):
                if f is not None:
                    f.check(cache.device, cache.n_layers, int(entries[i].pf.shape[1]), width, f"{name}[{i}]",
                            on_device=on_device)
    _on(block_table, cache.device, "block_table")
    ents = (kvr_rows * max(1, n))(*[e.c() for e in entries])
    pt = (ctypes.c_int64 * max(1, n))(*[int(x) for x in p_targets])

    def lr(lst, width, name):
        if lst is None:
            return None
        arr = (kvr_lowrank * max(1, n))()
        for i, f in enumerate(lst):
            if f is not None:
                arr[i] = f.c()
        return arr

    st = lib.kv_relocate_gather(ctypes.byref(cache.c), block_table.data_ptr(), int(block_table.numel()), ents,
                                pt, n, lr(patch_rope, int(cache.rope.shape[3]), "patch_rope"),
                                lr(patch_pf, int(cache.pf.shape[3]), "patch_pf"), _stream_handle())
    return _check("kv_relocate_gather", st)


def kv_patch_lowrank(cache, block_table, part, p_starts, lens, factors):
    """In-place X += U V^T on part 0 (position-free) or 1 (rotary) of the
    logical slots [p_starts[i], p_starts[i] + lens[i]) of every layer."""
    lib = _abi.load()
    n = len(factors)
    _i32(block_table, "block_table", 1)
    _need(part in (0, 1), "part must be 0 (position-free) or 1 (rotary)")
    _need(len(p_starts) == n and len(lens) == n, "p_starts and lens need one value per factor set")
    width = int((cache.rope if part else cache.pf).shape[3])
    for on_device in (False, True):
        for i, f in enumerate(factors):
            f.check(cache.device, cache.n_layers, int(lens[i]), width, f"factors[{i}]", on_device=on_device)
    _on(block_table, cache.device, "block_table")
    ps = (ctypes.c_int64 * max(1, n))(*[int(x) for x in p_starts])
    ln = (ctypes.c_int64 * max(1, n))(*[int(x) for x in lens])
    fs = (kvr_lowrank * max(1, n))(*[f.c() for f in factors])
    st = lib.kv_patch_lowrank(ctypes.byref(cache.c), block_table.data_ptr(), int(block_table.numel()), int(part),
                              ps, ln, fs, n, _stream_handle())
    return _check("kv_patch_lowrank", st)


def _decode_tables(device, b, block_tables, pending_delta, seq_lens, on_device):
    _i32(block_tables, "block_tables", 2, contiguous=False)
    _need(block_tables.stride(1) == 1, "block_tables needs a unit last stride")
    _need(int(block_tables.shape[0]) >= b, "block_tables needs a row per sequence")
    _i32(pending_delta, "pending_delta", 2, contiguous=False)
    _need(pending_delta.shape == block_tables.shape and pending_delta.stride() == block_tables.stride(),
          "pending_delta must match block_tables in shape and strides")
    _i32(seq_lens, "seq_lens", 1)
    _need(int(seq_lens.numel()) >= b, "seq_lens needs a length per sequence")
    if on_device:
        for t, nm in ((block_tables, "block_tables"), (pending_delta, "pending_delta"), (seq_lens, "seq_lens")):
            _on(t, device, nm)


def mla_decode_rotate_on_read(q_nope, q_rope, cache, layer, block_tables, pending_delta, seq_lens, scale,
                              max_seq_len=None, out=None, lse=None, workspace=None):
    """One absorbed-MLA decode step with per-block pending shifts applied to k_r on load.
    Returns (out bf16 [b, h, 512], lse f32 [b, h])."""
    lib = _abi.load()
    _need(q_nope.dim() == 3, "q_nope must be [batch, heads, 512]")
    b, h = int(q_nope.shape[0]), int(q_nope.shape[1])
    _tensor(q_nope, "q_nope", torch.bfloat16, (b, h, 512))
    _tensor(q_rope, "q_rope", torch.bfloat16, (b, h, 64))
    _decode_tables(cache.device, b, block_tables, pending_delta, seq_lens, False)
    if out is not None:
        _tensor(out, "out", torch.bfloat16, (b, h, 512))
    if lse is not None:
        _tensor(lse, "lse", torch.float32, (b, h))
    _decode_tables(cache.device, b, block_tables, pending_delta, seq_lens, True)
    for t, nm in ((q_nope, "q_nope"), (q_rope, "q_rope"), (out, "out"), (lse, "lse")):
        if t is not None:
            _on(t, cache.device, nm)
    if max_seq_len is None:
        max_seq_len = int(block_tables.shape[1]) * cache.block_size
    if out is None:
        out = torch.empty((b, h, 512), dtype=torch.bfloat16, device=q_nope.device)
    if lse is None:
        lse = torch.empty((b, h), dtype=torch.float32, device=q_nope.device)
    need = int(lib.kvr_decode_workspace_bytes(b, h, int(max_seq_len)))
    ws = workspace if workspace is not None else _workspace(need, q_nope.device, "decode")
    st = lib.mla_decode_rotate_on_read(q_nope.data_ptr(), q_rope.data_ptr(), b, h, ctypes.byref(cache.c), int(layer),
                                       block_tables.data_ptr(), pending_delta.data_ptr(), int(block_tables.stride(0)),
                                       seq_lens.data_ptr(), int(max_seq_len), float(scale), out.data_ptr(),
                                       lse.data_ptr(), ws.data_ptr(), ws.numel() * ws.element_size(),
                                       _stream_handle())
    _check("mla_decode_rotate_on_read", st)
    return out, lse


def gqa_decode_rotate_on_read(q, cache, layer, block_tables, pending_delta, seq_lens, scale,
                              max_seq_len=None, out=None, lse=None, workspace=None):
    """One GQA decode step over a paged cache (K = rope part, V = position-free
    part) with per-block pending shifts applied in attention.
    q: bf16 [b, q_heads, 128].  Returns (out bf16 [b, q_heads, 128], lse f32 [b, q_heads])."""
    lib = _abi.load()
    if q.dtype != torch.bfloat16 or q.dim() != 3 or not q.is_contiguous():
        raise ValueError("q must be a contiguous bf16 [batch, heads, dim] tensor")
    b, h = int(q.shape[0]), int(q.shape[1])
    kv = int(cache.c.rope_heads)
    _tensor(q, "q", torch.bfloat16, (b, h, 128))
    _decode_tables(cache.device, b, block_tables, pending_delta, seq_lens, False)
    if out is not None:
        _tensor(out, "out", torch.bfloat16, (b, h, 128))
    if lse is not None:
        _tensor(lse, "lse", torch.float32, (b, h))
    _decode_tables(cache.device, b, block_tables, pending_delta, seq_lens, True)
    for t, nm in ((q, "q"), (out, "out"), (lse, "lse")):
        if t is not None:
            _on(t, cache.device, nm)
    if max_seq_len is None:
        max_seq_len = int(block_tables.shape[1]) * cache.block_size
    if out is None:
        out = torch.empty((b, h, int(q.shape[2])), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((b, h), dtype=torch.float32, device=q.device)
    need = int(lib.kvr_gqa_decode_workspace_bytes(b, h, kv, int(max_seq_len)))
    ws = workspace if workspace is not None else _workspace(need, q.device, "gqa_decode")
    st = lib.gqa_decode_rotate_on_read(q.data_ptr(), b, h, ctypes.byref(cache.c), int(layer),
                                       block_tables.data_ptr(), pending_delta.data_ptr(), int(block_tables.stride(0)),
                                       seq_lens.data_ptr(), int(max_seq_len), float(scale), out.data_ptr(),
                                       lse.data_ptr(), ws.data_ptr(), ws.numel() * ws.element_size(),
                                       _stream_handle())
    _check("gqa_decode_rotate_on_read", st)
    return out, lse


def kamera_patch_factors(deficits, rank, omega, out=None, workspace=None):
    """Rank-m factors (U [n, rows, m] = U_m Sigma_m, V [n, cols, m], sigma
    [n, m]) of float32 deficits [n, rows, cols], or of the orbit mean of
    [n, orders, rows, cols]; omega: float32 [cols, 32] random test matrix."""
    lib = _abi.load()
    if deficits.dtype != torch.float32 or not deficits.is_contiguous() or deficits.dim() not in (3, 4):
        raise ValueError("deficits must be a contiguous float32 [n, (orders,) rows, cols] tensor")
    d4 = deficits if deficits.dim() == 4 else deficits.unsqueeze(1)
    n, orders, rows, cols = (int(x) for x in d4.shape)
    if omega.dtype != torch.float32 or not omega.is_contiguous() or tuple(omega.shape) != (cols, 32):
        raise ValueError("omega must be a contiguous float32 [cols, 32] tensor")
    dev = deficits.device
    if out is None:
        out = (torch.empty((n, rows, rank), dtype=torch.float32, device=dev),
               torch.empty((n, cols, rank), dtype=torch.float32, device=dev),
               torch.empty((n, rank), dtype=torch.float32, device=dev))
    U, V, s = out
    _tensor(U, "U", torch.float32, (n, rows, int(rank)))
    _tensor(V, "V", torch.float32, (n, cols, int(rank)))
    _tensor(s, "sigma", torch.float32, (n, int(rank)))
    for t, nm in ((deficits, "deficits"), (omega, "omega"), (U, "U"), (V, "V"), (s, "sigma")):
        _on(t, dev, nm)
    need = int(lib.kvr_patch_factors_workspace_bytes(n, orders, rows, cols))
    ws = workspace if workspace is not None else _workspace(need, dev, "form")
    st = lib.kamera_patch_factors(d4.data_ptr(), n, orders, rows, cols, int(rank), omega.data_ptr(), U.data_ptr(),
                                  V.data_ptr(), s.data_ptr(), ws.data_ptr(), ws.numel() * ws.element_size(),
                                  _stream_handle())
    _check("kamera_patch_factors", st)
    return U, V, s


def device_errors():
    """Synchronize and return (then clear) the library's device error bits.

    After a ticket or wait error of the ticketed splice, the cached splice
    workspaces may hold nonzero counters or stale flags; they are zeroed here,
    so that the next splice starts from a clean workspace."""
    lib = _abi.load()
    v = ctypes.c_uint32(0)
    _check("kvr_device_errors", lib.kvr_device_errors(ctypes.byref(v)))
    bits = int(v.value)
    if bits & (_abi.KVR_DEV_SPIN_LIMIT | _abi.KVR_DEV_BAD_TICKET):
        for key, ws in _workspaces.items():
            if key[0] == "splice":
                ws.zero_()
        torch.cuda.synchronize()
    return bits
