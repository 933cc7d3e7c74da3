"""ctypes view of libkvb.so (declarations mirror include/kvb.h)."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvb.so")

KVB_FP16 = 0
KVB_BF16 = 1

STATUS = {
    0: "KVB_OK",
    1: "KVB_ERR_NULL",
    2: "KVB_ERR_INVALID",
    3: "KVB_ERR_UNSUPPORTED",
    4: "KVB_ERR_WORKSPACE",
    5: "KVB_ERR_LAUNCH",
    6: "KVB_ERR_TOO_LARGE",
}

# every symbol include/kvb.h declares
EXPORTS = (
    "kvb_write_kv",
    "kvb_paged_prefill",
    "kvb_paged_prefill_write",
    "kvb_paged_prefill_pooled",
    "kvb_paged_decode",
    "kvb_paged_decode_noalloc",
    "kvb_paged_decode_cascade",
    "kvb_paged_prefill_workspace_size",
    "kvb_paged_decode_workspace_size",
    "kvb_paged_decode_cascade_workspace_size",
    "kvb_copy_blocks",
    "kvb_write_kv_q8",
    "kvb_paged_decode_q8",
    "kvb_paged_prefill_q8",
    "kvb_paged_prefill_q8_workspace_size",
    "kvb_write_kv_q4",
    "kvb_paged_decode_q4",
    "kvb_paged_prefill_q4",
    "kvb_gather_kv",
    "kvb_status_str",
    "kvb_version",
)


class KvbPool(ctypes.Structure):
    _fields_ = [
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("block_stride", ctypes.c_int64),
        ("num_blocks", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
    ]


class KvbPoolQ8(ctypes.Structure):
    _fields_ = [
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("v_scale", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p),
        ("block_stride", ctypes.c_int64),
        ("num_blocks", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
    ]


class KvbError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} failed: {STATUS.get(code, code)}")
        self.code = code


_lib = None

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_f32 = ctypes.c_float
_sz = ctypes.c_size_t
_PP = ctypes.POINTER(KvbPool)
_PQ = ctypes.POINTER(KvbPoolQ8)


def load() -> ctypes.CDLL:
    """Load libkvb.so; raises if it has not been built (there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build the HIP library first "
            "(python -m attention_paged_prefix_amd.build)")
    lib = ctypes.CDLL(LIB_PATH)
    lib.kvb_write_kv.argtypes = [_PP, _vp, _vp, _vp, _i32, _vp]
    lib.kvb_write_kv.restype = ctypes.c_int
    lib.kvb_paged_prefill.argtypes = [_PP, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32,
                                      _i32, _i32, _i32, _f32, _vp, _sz, _vp]
    lib.kvb_paged_prefill.restype = ctypes.c_int
    lib.kvb_paged_prefill_write.argtypes = [_PP, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32,
                                            _i32, _i32, _i32, _i32, _f32, _vp, _sz, _vp]
    lib.kvb_paged_prefill_write.restype = ctypes.c_int
    lib.kvb_paged_prefill_pooled.argtypes = [_PP, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                             _i32, _i32, _f32, _vp]
    lib.kvb_paged_prefill_pooled.restype = ctypes.c_int
    lib.kvb_paged_decode.argtypes = [_PP, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _f32,
                                     _vp, _sz, _vp]
    lib.kvb_paged_decode.restype = ctypes.c_int
    lib.kvb_paged_decode_noalloc.argtypes = [_PP, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                             _f32, _vp]
    lib.kvb_paged_decode_noalloc.restype = ctypes.c_int
    lib.kvb_paged_decode_cascade.argtypes = [_PP, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32,
                                             _i32, _i32, _f32, _vp, _sz, _vp]
    lib.kvb_paged_decode_cascade.restype = ctypes.c_int
    lib.kvb_paged_prefill_workspace_size.argtypes = [_i32, _i32, _i32, _i32, _i32]
    lib.kvb_paged_prefill_workspace_size.restype = _sz
    lib.kvb_paged_decode_workspace_size.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32]
    lib.kvb_paged_decode_workspace_size.restype = _sz
    lib.kvb_paged_decode_cascade_workspace_size.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32, _i32]
    lib.kvb_paged_decode_cascade_workspace_size.restype = _sz
    lib.kvb_copy_blocks.argtypes = [_PP, _PP, _vp, _vp, _i32, _vp]
    lib.kvb_copy_blocks.restype = ctypes.c_int
    lib.kvb_write_kv_q8.argtypes = [_PQ, _vp, _vp, _i32, _vp, _i32, _vp]
    lib.kvb_write_kv_q8.restype = ctypes.c_int
    lib.kvb_paged_decode_q8.argtypes = [_PQ, _i32, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                        _f32, _vp, _sz, _vp]
    lib.kvb_paged_decode_q8.restype = ctypes.c_int
    lib.kvb_paged_prefill_q8.argtypes = [_PQ, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32,
                                         _i32, _i32, _i32, _f32, _vp, _sz, _vp]
    lib.kvb_paged_prefill_q8.restype = ctypes.c_int
    lib.kvb_paged_prefill_q8_workspace_size.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32]
    lib.kvb_paged_prefill_q8_workspace_size.restype = _sz
    lib.kvb_write_kv_q4.argtypes = lib.kvb_write_kv_q8.argtypes
    lib.kvb_write_kv_q4.restype = ctypes.c_int
    lib.kvb_paged_decode_q4.argtypes = lib.kvb_paged_decode_q8.argtypes
    lib.kvb_paged_decode_q4.restype = ctypes.c_int
    lib.kvb_paged_prefill_q4.argtypes = lib.kvb_paged_prefill_q8.argtypes
    lib.kvb_paged_prefill_q4.restype = ctypes.c_int
    lib.kvb_gather_kv.argtypes = [_PP, _vp, _i32, _vp, _vp, _vp, _vp, _i32, _i32, _vp]
    lib.kvb_gather_kv.restype = ctypes.c_int
    lib.kvb_status_str.argtypes = [ctypes.c_int]
    lib.kvb_status_str.restype = ctypes.c_char_p
    lib.kvb_version.argtypes = []
    lib.kvb_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def check(fn: str, code: int) -> None:
    if code != 0:
        raise KvbError(fn, code)
