"""ctypes loader for libpkv.so; raises if the library has not been built."""

from __future__ import annotations

import ctypes
import os
import re

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libpkv.so")
HEADER = os.path.join(os.path.dirname(PKG_DIR), "include", "pkv.h")

PKV_OK = 0
PKV_ERR_INVALID_ARG = -1
PKV_ERR_OUT_OF_BLOCKS = -2
PKV_ERR_NO_SUCH_SEQ = -3
PKV_ERR_REFCOUNT = -4
PKV_ERR_UNSUPPORTED = -5
PKV_ERR_HIP = -6
PKV_ERR_WORKSPACE = -7
PKV_ERR_SWAPPED = -8
PKV_F32 = 0
PKV_BF16 = 1


class PkvError(RuntimeError):
    def __init__(self, status: int, call: str, msg: str):
        super().__init__(f"{call} failed: {msg} ({status})")
        self.status = status


class OutOfBlocks(PkvError):
    pass


class NoSuchSeq(PkvError):
    pass


class InvalidArg(PkvError):
    pass


class WrongTier(PkvError):
    """The sequence is swapped out (or, for a swap-in, is not)."""


class Stats(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int64) for name in (
        "num_blocks", "free_blocks", "used_blocks", "sum_refcount", "num_seqs",
        "logical_tokens", "logical_blocks", "allocated_slots", "table_bytes",
        "host_blocks", "host_free_blocks", "host_used_blocks", "swapped_seqs", "swapped_tokens",
        "cached_blocks", "cached_free_blocks")]

    def as_dict(self):
        return {name: int(getattr(self, name)) for name, _ in self._fields_}


i32, i64, vp, f32, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_size_t
P_i32 = ctypes.POINTER(ctypes.c_int32)
P_i64 = ctypes.POINTER(ctypes.c_int64)

_ATTN = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, f32, i32, vp, sz, i32, vp]

_SIGS = {
    "pkv_status_string": (ctypes.c_char_p, [i32]),
    "pkv_abi_version": (i32, []),
    "pkv_pool_create": (i32, [i32, i32, vp, ctypes.POINTER(vp)]),
    "pkv_pool_destroy": (None, [vp]),
    "pkv_seq_create": (i32, [vp, P_i32]),
    "pkv_seq_fork": (i32, [vp, i32, P_i32]),
    "pkv_seq_free": (i32, [vp, i32]),
    "pkv_append_tokens": (i32, [vp, vp, vp, i32, vp, vp, i64, vp, i32, P_i32]),
    "pkv_seq_create_prefixed": (i32, [vp, vp, i32, P_i32, P_i32]),
    "pkv_seq_truncate": (i32, [vp, i32, i32]),
    "pkv_pool_cached_blocks": (i32, [vp, vp, vp, i32, P_i32]),
    "pkv_block_tables": (i32, [vp, vp, i32, i32, vp, vp]),
    "pkv_seq_info": (i32, [vp, i32, P_i32, P_i32]),
    "pkv_pool_stats": (i32, [vp, ctypes.POINTER(Stats)]),
    "pkv_block_refcount": (i32, [vp, i32]),
    "pkv_pool_free_list": (i32, [vp, vp, i32, P_i32]),
    "pkv_pool_validate": (i32, [vp]),
    "pkv_pool_set_host_blocks": (i32, [vp, i32]),
    "pkv_swap_out": (i32, [vp, vp, i32, vp, i32, P_i32]),
    "pkv_swap_in": (i32, [vp, vp, i32, vp, i32, P_i32]),
    "pkv_seq_table": (i32, [vp, i32, vp, i32, P_i32, P_i32]),
    "pkv_host_block_refcount": (i32, [vp, i32]),
    "pkv_pool_host_free_list": (i32, [vp, vp, i32, P_i32]),
    "pkv_swap_blocks": (i32, [vp, vp, vp, vp, vp, i32, i32, i32, i64, vp]),
    "pkv_reshape_and_cache": (i32, [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp]),
    "pkv_copy_blocks": (i32, [vp, vp, vp, i32, i32, i64, vp]),
    "pkv_attention_workspace_bytes": (sz, [i32, i32, i32, i32, i32, i32, i32]),
    "pkv_hbm_read_probe": (i32, [vp, i64, vp, vp]),
    "pkv_paged_attention_decode": (i32, _ATTN),
    "pkv_paged_attention_partitions": (i32, _ATTN),
    "pkv_paged_attention_reduce": (i32, _ATTN),
    "pkv_decode_step": (i32, [vp, vp] + _ATTN),
    "pkv_decode_step_static": (i32, [vp, vp] + _ATTN[:16] + [i32, vp]),
    "pkv_paged_attention_multi": (i32, [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32,
                                        i32, i32, f32, vp, sz, i32, vp]),
    "pkv_attention_multi_workspace_bytes": (sz, [i32, i32, i32, i32, i32, i32]),
}

_lib = None


def header_symbols(path: str = HEADER):
    """Names of the functions pkv.h declares."""
    with open(path) as f:
        text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z0-9_]+)\s*\(", text)))


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m paged_kv_cache_physical_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def check(status: int, call: str) -> None:
    if status == PKV_OK:
        return
    msg = lib().pkv_status_string(status).decode()
    cls = {PKV_ERR_OUT_OF_BLOCKS: OutOfBlocks, PKV_ERR_NO_SUCH_SEQ: NoSuchSeq,
           PKV_ERR_INVALID_ARG: InvalidArg, PKV_ERR_SWAPPED: WrongTier}.get(status, PkvError)
    raise cls(status, call, msg)
