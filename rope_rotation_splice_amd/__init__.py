"""KV-cache relocation by closed-form RoPE delta-rotation on MI355X (gfx950).

The HIP library ``libkvreloc.so`` (C ABI in ``include/kvreloc.h``) does all
the work; this package marshals torch tensors into it.  Importing the package
loads the library and fails loudly if it has not been built.
"""

from . import _abi
from .api import (KVCache, KVRError, LowRank, Rows, device_errors, kv_patch_lowrank,  # noqa: F401
                  kv_relocate_gather, kv_relocate_gather_lazy, LazyBatch, LazyEntry, leyline_splice, leyline_splice_lazy,
                  leyline_splice_noalloc,
                  mla_decode_rotate_on_read, gqa_decode_rotate_on_read, kamera_patch_factors,
                  registry_chunk_keys,
                  splice_workspace_bytes,
                  KVR_AMORTIZE, KVR_FORGET, KVR_FORGET_NEEDS_PREFILL)

lib = _abi.load()
