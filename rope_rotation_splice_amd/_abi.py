"""ctypes mirror of include/kvreloc.h (argument marshalling only)."""

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkvreloc.so")

c_i32, c_i64, c_u32, c_f32, c_f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_float, ctypes.c_double
c_vp, c_size = ctypes.c_void_p, ctypes.c_size_t

KVR_OK = 0
KVR_FORGET_NEEDS_PREFILL = 1
KVR_E_WORKSPACE = -6
KVR_E_SCRATCH = -8
KVR_AMORTIZE, KVR_FORGET = 0, 1
KVR_BF16, KVR_F32 = 0, 1
KVR_DEV_BAD_BLOCK, KVR_DEV_SPIN_LIMIT, KVR_DEV_BAD_TICKET, KVR_DEV_RANGE, KVR_DEV_BAD_TOKEN = 1, 2, 4, 8, 16


class kvr_part(ctypes.Structure):
    _fields_ = [("base", c_vp), ("layer_stride", c_i64), ("block_stride", c_i64), ("row_stride", c_i64)]


class kvr_cache(ctypes.Structure):
    _fields_ = [("n_layers", c_i32), ("block_size", c_i32), ("n_blocks", c_i32), ("pf_width", c_i32),
                ("pf_dtype", c_i32), ("rope_heads", c_i32), ("rope_dim", c_i32), ("rope_dtype", c_i32),
                ("rope_base", c_f64), ("inv_freq", ctypes.POINTER(c_f64)), ("pf", kvr_part), ("rope", kvr_part)]


class kvr_directive(ctypes.Structure):
    _fields_ = [("s_start", c_i64), ("s_end", c_i64), ("r_len", c_i64), ("mode", c_i32), ("reserved", c_i32)]


class kvr_rows(ctypes.Structure):
    _fields_ = [("pf", c_vp), ("pf_layer_stride", c_i64), ("pf_row_stride", c_i64),
                ("rope", c_vp), ("rope_layer_stride", c_i64), ("rope_row_stride", c_i64),
                ("len", c_i64), ("base_pos", c_i64)]


class kvr_lowrank(ctypes.Structure):
    _fields_ = [("U", c_vp), ("u_layer_stride", c_i64), ("V", c_vp), ("v_layer_stride", c_i64),
                ("rank", c_i32), ("reserved", c_i32)]


class kvr_cdc_params(ctypes.Structure):
    _fields_ = [("threshold", ctypes.c_uint64), ("min_len", c_i32), ("max_len", c_i32), ("s1_window", c_i32),
                ("reserved", c_i32), ("seed", ctypes.c_uint64)]


class kvr_lazy_entry(ctypes.Structure):
    _fields_ = [("seq", c_i32), ("d_blocks", c_vp), ("d_pend", c_vp), ("len", c_i64), ("base_pos", c_i64),
                ("p_target", c_i64)]


P = ctypes.POINTER

# name -> (restype, argtypes); the names and order follow include/kvreloc.h
SIGNATURES = {
    "kvr_abi_version": (c_i32, []),
    "kvr_status_str": (ctypes.c_char_p, [c_i32]),
    "kvr_last_hip_error": (c_i32, []),
    "kvr_device_errors": (c_i32, [P(c_u32)]),
    "kvr_workspace_clear": (c_i32, [c_vp, c_size, c_vp]),
    "kvr_splice_workspace_bytes": (c_size, [P(kvr_cache), c_i32, P(c_i64), P(kvr_directive)]),
    "leyline_splice": (c_i32, [P(kvr_cache), c_vp, c_i32, c_i32, P(c_i64), P(kvr_directive), P(kvr_rows),
                               P(c_i64), c_vp, c_size, c_vp]),
    "leyline_splice_noalloc": (c_i32, [P(kvr_cache), c_vp, c_i32, c_i32, P(c_i64), P(kvr_directive), P(kvr_rows),
                                       P(c_i64), c_vp]),
    "kvr_noalloc_scratch_bytes": (c_size, []),
    "kv_relocate_gather": (c_i32, [P(kvr_cache), c_vp, c_i32, P(kvr_rows), P(c_i64), c_i32,
                                   P(kvr_lowrank), P(kvr_lowrank), c_vp]),
    "kv_patch_lowrank": (c_i32, [P(kvr_cache), c_vp, c_i32, c_i32, P(c_i64), P(c_i64), P(kvr_lowrank),
                                 c_i32, c_vp]),
    "kvr_decode_workspace_bytes": (c_size, [c_i32, c_i32, c_i32]),
    "mla_decode_rotate_on_read": (c_i32, [c_vp, c_vp, c_i32, c_i32, P(kvr_cache), c_i32, c_vp, c_vp, c_i32,
                                          c_vp, c_i32, c_f32, c_vp, c_vp, c_vp, c_size, c_vp]),
    "kvr_gqa_decode_workspace_bytes": (c_size, [c_i32, c_i32, c_i32, c_i32]),
    "gqa_decode_rotate_on_read": (c_i32, [c_vp, c_i32, c_i32, P(kvr_cache), c_i32, c_vp, c_vp, c_i32,
                                          c_vp, c_i32, c_f32, c_vp, c_vp, c_vp, c_size, c_vp]),
    "kvr_patch_factors_workspace_bytes": (c_size, [c_i32, c_i32, c_i32, c_i32]),
    "kamera_patch_factors": (c_i32, [c_vp, c_i32, c_i32, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_size,
                                     c_vp]),
    "leyline_splice_lazy": (c_i32, [c_i32, c_vp, c_vp, c_i32, c_i32, P(c_i64), P(kvr_directive), c_vp, c_vp,
                                    P(c_i64), c_vp]),
    "kv_relocate_gather_lazy": (c_i32, [c_i32, c_vp, c_vp, c_i32, c_i32, P(kvr_lazy_entry), c_i32, c_vp, c_vp]),
    "kvr_keys_workspace_bytes": (c_size, [c_i64]),
    "registry_chunk_keys": (c_i32, [c_vp, P(c_i64), c_i32, c_vp, c_i32, P(kvr_cdc_params), c_vp, c_vp, c_i32, c_vp,
                                    c_vp, c_vp, c_vp, c_size, c_vp]),
}

_lib = None


def load():
    """Load libkvreloc.so (built in-tree); fail loudly if it is missing.

    KVR_LIBRARY may name another build of the same library (the sanitized
    host build of the ABI check loads one this way)."""
    global _lib
    if _lib is not None:
        return _lib
    path = os.environ.get("KVR_LIBRARY") or LIB_PATH
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python rope_rotation_splice_amd/build.py`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.kvr_abi_version() != 1:
        raise ImportError("libkvreloc.so ABI version mismatch")
    _lib = lib
    return lib
