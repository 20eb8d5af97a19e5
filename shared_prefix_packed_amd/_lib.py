"""ctypes view of libpg.so (the C ABI in include/pg.h).

Loading fails loudly when the library has not been built: there is no
fallback path of any kind.
"""
from __future__ import annotations

import ctypes
import os

# PG_LIBRARY may name another build of the same library (the sanitizer build
# of the host code, python -m shared_prefix_packed_amd.build --sanitize).
LIB_PATH = os.environ.get("PG_LIBRARY") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libpg.so")

PG_OK = 0
PG_DECODE_SCRATCH_BYTES = 32 << 20   # include/pg.h
PG_F32 = 0
PG_BF16 = 1

c_int32 = ctypes.c_int32
c_int64 = ctypes.c_int64
c_void_p = ctypes.c_void_p
P_int32 = ctypes.POINTER(ctypes.c_int32)


class LayoutSummary(ctypes.Structure):
    _fields_ = [
        ("total_tokens", c_int64),
        ("num_groups", c_int32),
        ("num_segments", c_int32),
        ("max_position", c_int32),
        ("num_items", c_int32),
        ("num_spans", c_int32),
        ("block_tokens", c_int32),
        ("heads_per_item", c_int32),
        ("device_ready", c_int32),
        ("useful_pairs", c_int64),
        ("unpacked_pairs", c_int64),
        ("max_item_cost", c_int64),
        ("max_xcd_cost", c_int64),
        ("num_kv_items", c_int32),
        ("num_dec_items", c_int32),
        ("num_dec_refs", ctypes.c_int64),
        ("max_group_len", c_int32),
        ("reserved", c_int32),
    ]


class WorkItem(ctypes.Structure):
    _fields_ = [("t0", c_int32), ("t1", c_int32), ("hq0", c_int32), ("pe", c_int32),
                ("span0", c_int32), ("nspan", c_int32), ("ntiles", c_int32),
                ("k0", c_int32), ("k1", c_int32), ("reserved", c_int32), ("cost", c_int64)]


class KeySpan(ctypes.Structure):
    _fields_ = [("k0", c_int32), ("k1", c_int32)]


class DecItem(ctypes.Structure):
    _fields_ = [("k0", c_int32), ("k1", c_int32), ("hk", c_int32), ("resp", c_int32),
                ("seg0", c_int32), ("seg1", c_int32), ("row0", c_int32), ("nrow", c_int32)]


class KvItem(ctypes.Structure):
    _fields_ = [("k0", c_int32), ("k1", c_int32), ("hk", c_int32), ("qend", c_int32),
                ("cost", c_int64)]


# name -> (restype, argtypes); every symbol include/pg.h declares
SIGNATURES = {
    "pg_build_layout_host": (c_int32, [c_int32, P_int32, P_int32, P_int32, c_int32, c_int32,
                                       c_int32, ctypes.c_double, ctypes.POINTER(c_void_p)]),
    "pg_layout_upload": (c_int32, [c_void_p, c_void_p]),
    "pg_build_layout": (c_int32, [c_int32, P_int32, P_int32, P_int32, c_int32, c_int32, c_int32,
                                  ctypes.c_double, c_void_p, ctypes.POINTER(c_void_p)]),
    "pg_layout_info": (c_int32, [c_void_p, ctypes.POINTER(LayoutSummary)]),
    "pg_layout_copy_offsets": (c_int32, [c_void_p, P_int32, P_int32]),
    "pg_layout_copy_tokens": (c_int32, [c_void_p, P_int32, P_int32, P_int32]),
    "pg_layout_copy_work": (c_int32, [c_void_p, ctypes.POINTER(WorkItem),
                                      ctypes.POINTER(KeySpan)]),
    "pg_layout_copy_kv_work": (c_int32, [c_void_p, ctypes.POINTER(KvItem)]),
    "pg_layout_copy_decode_work": (c_int32, [c_void_p, ctypes.POINTER(DecItem), P_int32, P_int32]),
    "pg_decode_workspace_size": (c_int32, [c_void_p, ctypes.POINTER(ctypes.c_size_t)]),
    "pg_attn_decode": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                 c_void_p, c_void_p, ctypes.c_size_t, c_int32, ctypes.c_float,
                                 c_void_p]),
    "pg_attn_decode_noalloc": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                         c_void_p, c_void_p, c_int32, ctypes.c_float, c_void_p]),
    "pg_layout_destroy": (None, [c_void_p]),
    "pg_position_ids": (c_int32, [c_void_p, c_void_p, c_void_p]),
    "pg_rope": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int32,
                          c_void_p]),
    "pg_attn_fwd": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                              c_int32, ctypes.c_float, c_void_p]),
    "pg_attn_bwd": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                              c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int32,
                              ctypes.c_float, c_void_p]),
    "pg_pack_rows": (c_int32, [c_void_p, c_void_p, c_int32, c_void_p, c_int32, c_void_p,
                               ctypes.c_int64, c_void_p]),
    "pg_unpack_rows": (c_int32, [c_void_p, c_void_p, ctypes.c_int64, c_void_p, c_int32,
                                 c_void_p, c_int32, c_void_p]),
    "pg_position_ids_padded": (c_int32, [c_void_p, c_int32, c_void_p, c_void_p, c_void_p]),
    "pg_pad_rows": (c_int32, [c_void_p, c_void_p, ctypes.c_int64, c_void_p, c_int32, c_void_p]),
    "pg_unpad_rows": (c_int32, [c_void_p, c_void_p, c_int32, ctypes.c_int64, c_void_p, c_void_p]),
    "pg_status_string": (ctypes.c_char_p, [c_int32]),
    "pg_last_error": (ctypes.c_char_p, []),
}

_lib = None


def load() -> ctypes.CDLL:
    """Load libpg.so once. Raises if it is missing or lacks a symbol."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built; run `python -m shared_prefix_packed_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class PgError(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = load()
        text = lib.pg_status_string(status).decode()
        detail = lib.pg_last_error().decode()
        super().__init__(f"{where}: {text} ({status}): {detail}")
        self.status = status


def check(status: int, where: str) -> None:
    if status != PG_OK:
        raise PgError(status, where)
