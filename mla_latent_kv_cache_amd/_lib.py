"""ctypes view of libmla_kv.so: the C ABI declared in include/mla_kv.h.

Argument marshalling only. Every step of the decode path runs in the HIP
library; if the library is missing this module raises instead of falling
back to anything else.
"""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmla_kv.so")

MLA_OK = 0
MLA_ERR_INVALID_ARG = -1
MLA_ERR_UNSUPPORTED = -2
MLA_ERR_WORKSPACE = -3
MLA_ERR_CAPACITY = -4
MLA_ERR_HIP = -5
STATIC_SCRATCH_BYTES = 64 << 20  # MLA_STATIC_SCRATCH_BYTES of include/mla_kv.h

FORMATS = {"bf16": 0, "int8": 1, "int4": 2, "int8_kbf16": 3, "int4_kint4": 4}

# Every symbol include/mla_kv.h declares.
SYMBOLS = (
    "mla_cache_append",
    "mla_decode_workspace_bytes",
    "mla_decode_auto_splits",
    "mla_decode_attn",
    "mla_decode_step",
    "mla_decode_workspace_bytes_layers",
    "mla_decode_auto_splits_layers",
    "mla_decode_attn_layers",
    "mla_decode_step_layers",
    "mla_decode_step_begin_layers",
    "mla_decode_absorb_layers",
    "mla_decode_partial_layers",
    "mla_decode_combine_layers",
    "mla_stream_read",
    "mla_mfma_rate",
    "mla_decode_attn_static",
    "mla_decode_step_begin",
    "mla_decode_absorb",
    "mla_decode_partial",
    "mla_decode_combine",
    "mla_cache_get",
    "mla_rope_tables",
    "mla_status_str",
)


class MlaCacheStruct(ctypes.Structure):
    """Mirror of `struct mla_cache`."""
    _fields_ = [
        ("format", ctypes.c_int32),
        ("num_layers", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("capacity", ctypes.c_int32),
        ("kv_lora_rank", ctypes.c_int32),
        ("rope_dim", ctypes.c_int32),
        ("group_latent", ctypes.c_int32),
        ("group_rope", ctypes.c_int32),
        ("ckv", ctypes.c_void_p),
        ("kpe", ctypes.c_void_p),
        ("scale", ctypes.c_void_p),
        ("zero", ctypes.c_void_p),
        ("seq_lens", ctypes.c_void_p),
        ("page_size", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("block_table", ctypes.c_void_p),
    ]


class MlaError(RuntimeError):
    def __init__(self, status, where=""):
        self.status = status
        msg = status_str(status) if _lib is not None else str(status)
        super().__init__(f"{where}: {msg} (status {status})" if where else f"{msg} (status {status})")


_lib = None


def lib():
    """Load the HIP library (once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build() first")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(MlaCacheStruct)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        L.mla_cache_append.argtypes = [P, i32, vp, vp, i32, vp, vp]
        L.mla_cache_append.restype = ctypes.c_int
        L.mla_decode_workspace_bytes.argtypes = [P, i32, i32, ctypes.POINTER(sz)]
        L.mla_decode_workspace_bytes.restype = ctypes.c_int
        L.mla_decode_auto_splits.argtypes = [P, i32, ctypes.POINTER(i32)]
        L.mla_decode_auto_splits.restype = ctypes.c_int
        L.mla_decode_attn.argtypes = [P, i32, vp, vp, vp, vp, i32, ctypes.c_float, i32, vp, sz, vp, vp]
        L.mla_decode_attn.restype = ctypes.c_int
        L.mla_decode_step.argtypes = [P, i32, vp, vp, vp, vp, vp, vp, i32, vp, vp, i32, ctypes.c_float, i32,
                                      vp, sz, vp, vp]
        L.mla_decode_step.restype = ctypes.c_int
        L.mla_decode_workspace_bytes_layers.argtypes = [P, i32, i32, i32, ctypes.POINTER(sz)]
        L.mla_decode_workspace_bytes_layers.restype = ctypes.c_int
        L.mla_decode_auto_splits_layers.argtypes = [P, i32, i32, ctypes.POINTER(i32)]
        L.mla_decode_auto_splits_layers.restype = ctypes.c_int
        L.mla_decode_attn_layers.argtypes = [P, i32, i32, vp, vp, vp, vp, i32, ctypes.c_float, i32, vp, sz, vp,
                                             vp]
        L.mla_decode_attn_layers.restype = ctypes.c_int
        L.mla_decode_step_layers.argtypes = [P, i32, i32, vp, vp, vp, vp, vp, vp, i32, vp, vp, i32,
                                             ctypes.c_float, i32, vp, sz, vp, vp]
        L.mla_decode_step_layers.restype = ctypes.c_int
        L.mla_decode_step_begin_layers.argtypes = [P, i32, i32, vp, vp, vp, vp, vp, vp, i32, vp, i32,
                                                   ctypes.c_float, i32, vp, sz, vp]
        L.mla_decode_step_begin_layers.restype = ctypes.c_int
        L.mla_decode_absorb_layers.argtypes = [P, i32, vp, vp, vp, i32, ctypes.c_float, i32, vp, sz, vp]
        L.mla_decode_absorb_layers.restype = ctypes.c_int
        L.mla_decode_partial_layers.argtypes = [P, i32, i32, i32, i32, vp, sz, vp]
        L.mla_decode_partial_layers.restype = ctypes.c_int
        L.mla_decode_combine_layers.argtypes = [P, i32, vp, i32, i32, vp, sz, vp, vp]
        L.mla_decode_combine_layers.restype = ctypes.c_int
        L.mla_decode_attn_static.argtypes = [P, i32, vp, vp, vp, vp, i32, ctypes.c_float, i32, vp, vp]
        L.mla_decode_attn_static.restype = ctypes.c_int
        L.mla_stream_read.argtypes = [vp, sz, vp, i32, i32, vp]
        L.mla_stream_read.restype = ctypes.c_int
        L.mla_mfma_rate.argtypes = [vp, i32, i32, vp]
        L.mla_mfma_rate.restype = ctypes.c_int
        L.mla_decode_step_begin.argtypes = [P, i32, vp, vp, vp, vp, vp, vp, i32, vp, i32, ctypes.c_float, i32,
                                            vp, sz, vp]
        L.mla_decode_step_begin.restype = ctypes.c_int
        L.mla_decode_absorb.argtypes = [P, vp, vp, vp, i32, ctypes.c_float, i32, vp, sz, vp]
        L.mla_decode_absorb.restype = ctypes.c_int
        L.mla_decode_partial.argtypes = [P, i32, i32, i32, vp, sz, vp]
        L.mla_decode_partial.restype = ctypes.c_int
        L.mla_decode_combine.argtypes = [P, vp, i32, i32, vp, sz, vp, vp]
        L.mla_decode_combine.restype = ctypes.c_int
        L.mla_cache_get.argtypes = [P, i32, vp, vp, vp]
        L.mla_cache_get.restype = ctypes.c_int
        L.mla_rope_tables.argtypes = [vp, vp, i32, ctypes.c_double, vp]
        L.mla_rope_tables.restype = ctypes.c_int
        L.mla_status_str.argtypes = [ctypes.c_int]
        L.mla_status_str.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_str(status):
    return lib().mla_status_str(int(status)).decode()


def check(status, where=""):
    if status != MLA_OK:
        raise MlaError(status, where)
    return status
