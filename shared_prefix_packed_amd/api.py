"""Thin Python binding of libpg.so: the same entry points as include/pg.h.

Only argument marshalling happens here (shape/dtype checks, raw pointers,
the current torch stream). Every step of the path runs in the library.
torch is used for device memory and streams only.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence, Tuple

import numpy as np

from . import _lib
from ._lib import DecItem, KeySpan, KvItem, LayoutSummary, WorkItem, check, load


def _i32(x) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(x, dtype=np.int64))
    if a.size and (a.min() < -(2**31) or a.max() >= 2**31):
        raise ValueError("length does not fit int32")
    return np.ascontiguousarray(a.astype(np.int32))


def _ptr_i32(a: np.ndarray):
    return a.ctypes.data_as(_lib.P_int32) if a.size else None


def _stream_handle(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


class Layout:
    """Owner of one pg_layout handle (freed on close / garbage collection)."""

    def __init__(self, handle: int, heads: Tuple[int, int, int]):
        self._h = ctypes.c_void_p(handle)
        self.num_q_heads, self.num_kv_heads, self.head_dim = heads

    @property
    def handle(self) -> ctypes.c_void_p:
        if not self._h:
            raise ValueError("layout is closed")
        return self._h

    def close(self) -> None:
        if self._h:
            load().pg_layout_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def summary(self) -> LayoutSummary:
        s = LayoutSummary()
        check(load().pg_layout_info(self.handle, ctypes.byref(s)), "pg_layout_info")
        return s

    @property
    def total_tokens(self) -> int:
        return int(self.summary().total_tokens)

    def offsets(self) -> Tuple[np.ndarray, np.ndarray]:
        s = self.summary()
        g = np.zeros(s.num_groups + 1, dtype=np.int32)
        seg = np.zeros(s.num_segments + 1, dtype=np.int32)
        check(load().pg_layout_copy_offsets(self.handle, _ptr_i32(g), _ptr_i32(seg)),
              "pg_layout_copy_offsets")
        return g, seg

    def tokens(self) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
        T = self.total_tokens
        g0, pe, ss = (np.zeros(T, dtype=np.int32) for _ in range(3))
        check(load().pg_layout_copy_tokens(self.handle, _ptr_i32(g0), _ptr_i32(pe), _ptr_i32(ss)),
              "pg_layout_copy_tokens")
        return g0, pe, ss

    def work(self) -> Tuple[np.ndarray, np.ndarray]:
        """Work items (structured array, launch order) and key spans [n, 2]."""
        s = self.summary()
        items = (WorkItem * max(1, s.num_items))()
        spans = (KeySpan * max(1, s.num_spans))()
        check(load().pg_layout_copy_work(self.handle, items, spans), "pg_layout_copy_work")
        it = np.frombuffer(items, dtype=np.dtype([("t0", "<i4"), ("t1", "<i4"), ("hq0", "<i4"),
                                                  ("pe", "<i4"), ("span0", "<i4"),
                                                  ("nspan", "<i4"), ("ntiles", "<i4"),
                                                  ("k0", "<i4"), ("k1", "<i4"),
                                                  ("reserved", "<i4"), ("cost", "<i8")]))
        sp = np.frombuffer(spans, dtype=np.int32).reshape(-1, 2)
        return it[:s.num_items].copy(), sp[:s.num_spans].copy()

    def kv_work(self) -> np.ndarray:
        """Backward dK/dV work items (structured array, launch order)."""
        s = self.summary()
        items = (KvItem * max(1, s.num_kv_items))()
        check(load().pg_layout_copy_kv_work(self.handle, items), "pg_layout_copy_kv_work")
        it = np.frombuffer(items, dtype=np.dtype([("k0", "<i4"), ("k1", "<i4"), ("hk", "<i4"),
                                                  ("qend", "<i4"), ("cost", "<i8")]))
        return it[:s.num_kv_items].copy()

    @property
    def num_responses(self) -> int:
        s = self.summary()
        return s.num_segments - s.num_groups

    def decode_work(self) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
        """Decode work items (structured array, launch order), the merge-list
        offsets [N * Hkv + 1] and the merge lists (item indices)."""
        s = self.summary()
        n_off = self.num_responses * self.num_kv_heads + 1
        items = (DecItem * max(1, s.num_dec_items))()
        off = np.zeros(max(1, n_off), dtype=np.int32)
        refs = np.zeros(max(1, s.num_dec_refs), dtype=np.int32)
        check(load().pg_layout_copy_decode_work(self.handle, items, _ptr_i32(off), _ptr_i32(refs)),
              "pg_layout_copy_decode_work")
        it = np.frombuffer(items, dtype=np.dtype([(n, "<i4") for n in
                                                  ("k0", "k1", "hk", "resp", "seg0", "seg1",
                                                   "row0", "nrow")]))
        return it[:s.num_dec_items].copy(), off[:n_off].copy(), refs[:s.num_dec_refs].copy()

    def decode_workspace_size(self) -> int:
        """Bytes of device scratch pg_attn_decode needs on this layout."""
        n = ctypes.c_size_t(0)
        check(load().pg_decode_workspace_size(self.handle, ctypes.byref(n)),
              "pg_decode_workspace_size")
        return int(n.value)


def _layout_args(prefix_lens, suffix_counts, suffix_lens):
    P, n, S = _i32(prefix_lens), _i32(suffix_counts), _i32(suffix_lens)
    if P.shape != n.shape:
        raise ValueError("prefix_lens and suffix_counts differ in length")
    return P, n, S


def pg_build_layout_host(prefix_lens: Sequence[int], suffix_counts: Sequence[int],
                         suffix_lens: Sequence[int], num_q_heads: int, num_kv_heads: int,
                         head_dim: int, rope_theta: float) -> Layout:
    P, n, S = _layout_args(prefix_lens, suffix_counts, suffix_lens)
    out = ctypes.c_void_p()
    check(load().pg_build_layout_host(len(P), _ptr_i32(P), _ptr_i32(n), _ptr_i32(S),
                                      num_q_heads, num_kv_heads, head_dim, float(rope_theta),
                                      ctypes.byref(out)), "pg_build_layout_host")
    return Layout(out.value, (num_q_heads, num_kv_heads, head_dim))


def pg_layout_upload(layout: Layout, stream=None) -> None:
    check(load().pg_layout_upload(layout.handle, _stream_handle(stream)), "pg_layout_upload")


def pg_build_layout(prefix_lens: Sequence[int], suffix_counts: Sequence[int],
                    suffix_lens: Sequence[int], num_q_heads: int, num_kv_heads: int,
                    head_dim: int, rope_theta: float, stream=None) -> Layout:
    P, n, S = _layout_args(prefix_lens, suffix_counts, suffix_lens)
    out = ctypes.c_void_p()
    check(load().pg_build_layout(len(P), _ptr_i32(P), _ptr_i32(n), _ptr_i32(S), num_q_heads,
                                 num_kv_heads, head_dim, float(rope_theta),
                                 _stream_handle(stream), ctypes.byref(out)), "pg_build_layout")
    return Layout(out.value, (num_q_heads, num_kv_heads, head_dim))


# ------------------------------------------------------------ device calls --

def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return _lib.PG_BF16
    if t.dtype == torch.float32:
        return _lib.PG_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _check_tensor(name, t, shape, dtype=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on the GPU")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def pg_position_ids(layout: Layout, pos=None, stream=None):
    """int64 [T] position ids on the current device."""
    import torch
    T = layout.total_tokens
    if pos is None:
        pos = torch.empty(T, dtype=torch.int64, device="cuda")
    _check_tensor("pos", pos, (T,), torch.int64)
    check(load().pg_position_ids(layout.handle, ctypes.c_void_p(pos.data_ptr()),
                                 _stream_handle(stream)), "pg_position_ids")
    return pos


def pg_rope(layout: Layout, pos, q, k, q_out=None, k_out=None, stream=None):
    """RoPE of q [T, Hq, d] and k [T, Hkv, d] at `pos`; out-of-place unless
    q_out is q / k_out is k. q or k may be None: only the other is rotated
    (the returned output for the missing one is None)."""
    import torch
    T, Hq, Hkv, d = layout.total_tokens, layout.num_q_heads, layout.num_kv_heads, layout.head_dim
    if q is None and k is None:
        raise ValueError("nothing to rotate")
    _check_tensor("pos", pos, (T,), torch.int64)
    ref = q if q is not None else k
    if q is not None:
        _check_tensor("q", q, (T, Hq, d))
        if q_out is None:
            q_out = torch.empty_like(q)
        _check_tensor("q_out", q_out, (T, Hq, d), ref.dtype)
    else:
        q_out = None
    if k is not None:
        _check_tensor("k", k, (T, Hkv, d), ref.dtype)
        if k_out is None:
            k_out = torch.empty_like(k)
        _check_tensor("k_out", k_out, (T, Hkv, d), ref.dtype)
    else:
        k_out = None
    ptr = lambda t: ctypes.c_void_p(t.data_ptr() if t is not None else None)
    check(load().pg_rope(layout.handle, ptr(pos), ptr(q), ptr(k), ptr(q_out), ptr(k_out),
                         _dtype_code(ref), _stream_handle(stream)), "pg_rope")
    return q_out, k_out


def pg_attn_fwd(layout: Layout, q, k, v, softmax_scale: float, o=None, lse=None,
                want_lse: bool = True, stream=None):
    """Packed attention forward. Returns (o [T, Hq, d], lse fp32 [Hq, T] or None)."""
    import torch
    T, Hq, Hkv, d = layout.total_tokens, layout.num_q_heads, layout.num_kv_heads, layout.head_dim
    _check_tensor("q", q, (T, Hq, d))
    _check_tensor("k", k, (T, Hkv, d), q.dtype)
    _check_tensor("v", v, (T, Hkv, d), q.dtype)
    if o is None:
        o = torch.empty_like(q)
    _check_tensor("o", o, (T, Hq, d), q.dtype)
    if lse is None and want_lse:
        lse = torch.empty((Hq, T), dtype=torch.float32, device=q.device)
    if lse is not None:
        _check_tensor("lse", lse, (Hq, T), torch.float32)
    check(load().pg_attn_fwd(layout.handle, ctypes.c_void_p(q.data_ptr()),
                             ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
                             ctypes.c_void_p(o.data_ptr()),
                             ctypes.c_void_p(lse.data_ptr() if lse is not None else None),
                             _dtype_code(q), float(softmax_scale), _stream_handle(stream)),
          "pg_attn_fwd")
    return o, lse


def pg_attn_bwd(layout: Layout, q, k, v, o, lse, dout, softmax_scale: float, dq=None, dk=None,
                dv=None, delta=None, stream=None):
    """Packed attention backward for an upstream gradient dout of the forward's
    o (lse: the forward's fp32 [Hq, T]). Returns (dq, dk, dv)."""
    import torch
    T, Hq, Hkv, d = layout.total_tokens, layout.num_q_heads, layout.num_kv_heads, layout.head_dim
    _check_tensor("q", q, (T, Hq, d))
    _check_tensor("k", k, (T, Hkv, d), q.dtype)
    _check_tensor("v", v, (T, Hkv, d), q.dtype)
    _check_tensor("o", o, (T, Hq, d), q.dtype)
    _check_tensor("dout", dout, (T, Hq, d), q.dtype)
    _check_tensor("lse", lse, (Hq, T), torch.float32)
    if dq is None:
        dq = torch.empty_like(q)
    if dk is None:
        dk = torch.empty_like(k)
    if dv is None:
        dv = torch.empty_like(v)
    if delta is None:
        delta = torch.empty((Hq, T), dtype=torch.float32, device=q.device)
    _check_tensor("dq", dq, (T, Hq, d), q.dtype)
    _check_tensor("dk", dk, (T, Hkv, d), q.dtype)
    _check_tensor("dv", dv, (T, Hkv, d), q.dtype)
    _check_tensor("delta", delta, (Hq, T), torch.float32)
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())
    check(load().pg_attn_bwd(layout.handle, ptr(q), ptr(k), ptr(v), ptr(o), ptr(lse), ptr(dout),
                             ptr(dq), ptr(dk), ptr(dv), ptr(delta), _dtype_code(q),
                             float(softmax_scale), _stream_handle(stream)),
          "pg_attn_bwd")
    return dq, dk, dv


def pg_attn_decode(layout: Layout, q, k_cache, v_cache, cur_lens, softmax_scale: float, o=None,
                   lse=None, workspace=None, stream=None):
    """One decode step over a group-contiguous KV cache laid out as ``layout``
    (response segments at capacity). q: [N, Hq, d], one query per response;
    cur_lens: device int32 [N]. Returns (o [N, Hq, d], lse fp32 [Hq, N])."""
    import torch
    T, Hq, Hkv, d = layout.total_tokens, layout.num_q_heads, layout.num_kv_heads, layout.head_dim
    N = layout.num_responses
    _check_tensor("q", q, (N, Hq, d))
    _check_tensor("k_cache", k_cache, (T, Hkv, d), q.dtype)
    _check_tensor("v_cache", v_cache, (T, Hkv, d), q.dtype)
    _check_tensor("cur_lens", cur_lens, (N,), torch.int32)
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((Hq, N), dtype=torch.float32, device=q.device)
    _check_tensor("o", o, (N, Hq, d), q.dtype)
    _check_tensor("lse", lse, (Hq, N), torch.float32)
    need = layout.decode_workspace_size()
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    if workspace.device.type != "cuda" or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    ws_bytes = workspace.numel() * workspace.element_size()
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())
    check(load().pg_attn_decode(layout.handle, ptr(q), ptr(k_cache), ptr(v_cache), ptr(cur_lens),
                                ptr(o), ptr(lse), ptr(workspace), ctypes.c_size_t(ws_bytes),
                                _dtype_code(q), float(softmax_scale), _stream_handle(stream)),
          "pg_attn_decode")
    return o, lse


def pg_attn_decode_noalloc(layout: Layout, q, k_cache, v_cache, cur_lens, softmax_scale: float,
                           o=None, lse=None, stream=None):
    """pg_attn_decode without a workspace: the library keeps the partial
    results in its static per-GPU scratch array. The C call allocates
    nothing; pass o and lse to allocate nothing here either."""
    import torch
    T, Hq, Hkv, d = layout.total_tokens, layout.num_q_heads, layout.num_kv_heads, layout.head_dim
    N = layout.num_responses
    _check_tensor("q", q, (N, Hq, d))
    _check_tensor("k_cache", k_cache, (T, Hkv, d), q.dtype)
    _check_tensor("v_cache", v_cache, (T, Hkv, d), q.dtype)
    _check_tensor("cur_lens", cur_lens, (N,), torch.int32)
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((Hq, N), dtype=torch.float32, device=q.device)
    _check_tensor("o", o, (N, Hq, d), q.dtype)
    _check_tensor("lse", lse, (Hq, N), torch.float32)
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())
    check(load().pg_attn_decode_noalloc(layout.handle, ptr(q), ptr(k_cache), ptr(v_cache),
                                        ptr(cur_lens), ptr(o), ptr(lse), _dtype_code(q),
                                        float(softmax_scale), _stream_handle(stream)),
          "pg_attn_decode_noalloc")
    return o, lse


def _row_bytes(t, lead: int) -> int:
    n = 1
    for x in t.shape[lead:]:
        n *= int(x)
    return n * t.element_size()


def pg_pack_rows(layout: Layout, prefix, suffix, packed=None, stream=None):
    """Packed rows [T, ...] from right-padded prompts [G, Ppad, ...] and
    responses [N, Spad, ...] (any dtype; rows of a multiple of 4 bytes)."""
    import torch
    if not (prefix.is_contiguous() and suffix.is_contiguous()):
        raise ValueError("prefix and suffix must be contiguous")
    if prefix.dtype != suffix.dtype or prefix.shape[2:] != suffix.shape[2:]:
        raise ValueError("prefix and suffix rows differ")
    T = layout.total_tokens
    if packed is None:
        packed = torch.empty((T,) + tuple(prefix.shape[2:]), dtype=prefix.dtype, device=prefix.device)
    check(load().pg_pack_rows(layout.handle, ctypes.c_void_p(prefix.data_ptr()), int(prefix.shape[1]),
                              ctypes.c_void_p(suffix.data_ptr()), int(suffix.shape[1]),
                              ctypes.c_void_p(packed.data_ptr()), _row_bytes(prefix, 2),
                              _stream_handle(stream)),
          "pg_pack_rows")
    return packed


def pg_unpack_rows(layout: Layout, packed, prefix_pad: int, suffix_pad: int, prefix_out=None,
                   suffix_out=None, stream=None):
    """(prefix_out [G, prefix_pad, ...], suffix_out [N, suffix_pad + 1, ...]):
    the packed rows split back, each response part led by its group's last
    prompt row. Outputs given by the caller are filled in place (nothing is
    allocated then, as under graph capture)."""
    import torch
    if not packed.is_contiguous():
        raise ValueError("packed must be contiguous")
    s = layout.summary()
    n_resp = int(np.asarray(layout.offsets()[1]).size - 1 - s.num_groups)
    tail = tuple(packed.shape[1:])
    pre_shape = (s.num_groups, prefix_pad) + tail
    suf_shape = (n_resp, suffix_pad + 1) + tail
    pre = prefix_out if prefix_out is not None else torch.empty(pre_shape, dtype=packed.dtype,
                                                                device=packed.device)
    suf = suffix_out if suffix_out is not None else torch.empty(suf_shape, dtype=packed.dtype,
                                                                device=packed.device)
    _check_tensor("prefix_out", pre, pre_shape, packed.dtype)
    _check_tensor("suffix_out", suf, suf_shape, packed.dtype)
    check(load().pg_unpack_rows(layout.handle, ctypes.c_void_p(packed.data_ptr()),
                                _row_bytes(packed, 1), ctypes.c_void_p(pre.data_ptr()),
                                int(prefix_pad), ctypes.c_void_p(suf.data_ptr()), int(suffix_pad),
                                _stream_handle(stream)),
          "pg_unpack_rows")
    return pre, suf


# ------------------------------------------------- right-padded form --

def _max_len(layout: Layout, max_len) -> int:
    return layout.summary().max_group_len if max_len is None else int(max_len)


def pg_position_ids_padded(layout: Layout, max_len: Optional[int] = None, stream=None):
    """Position ids (int64) and padding mask (uint8) of the right-padded form
    [G, max_len]; max_len defaults to the longest group row."""
    import torch
    G, L = layout.summary().num_groups, _max_len(layout, max_len)
    pos = torch.empty((G, L), dtype=torch.int64, device="cuda")
    mask = torch.empty((G, L), dtype=torch.uint8, device="cuda")
    ptr = lambda t: ctypes.c_void_p(t.data_ptr() if t.numel() else None)
    check(load().pg_position_ids_padded(layout.handle, L, ptr(pos), ptr(mask),
                                        _stream_handle(stream)), "pg_position_ids_padded")
    return pos, mask


def pg_pad_rows(layout: Layout, packed, max_len: Optional[int] = None, padded=None, stream=None):
    """Packed rows [T, ...] to the right-padded form [G, max_len, ...]
    (max_len: that of ``padded`` if given, else the longest group row)."""
    import torch
    if max_len is None and padded is not None and padded.dim() >= 2:
        max_len = padded.shape[1]
    G, L = layout.summary().num_groups, _max_len(layout, max_len)
    _check_tensor("packed", packed, (layout.total_tokens,) + tuple(packed.shape[1:]))
    rb = _row_bytes(packed, 1)
    if padded is None:
        padded = torch.empty((G, L) + tuple(packed.shape[1:]), dtype=packed.dtype, device="cuda")
    _check_tensor("padded", padded, (G, L) + tuple(packed.shape[1:]), packed.dtype)
    ptr = lambda t: ctypes.c_void_p(t.data_ptr() if t.numel() else None)
    check(load().pg_pad_rows(layout.handle, ptr(packed), ctypes.c_int64(rb), ptr(padded), L,
                             _stream_handle(stream)), "pg_pad_rows")
    return padded


def pg_unpad_rows(layout: Layout, padded, packed=None, stream=None):
    """The right-padded form [G, max_len, ...] back to packed rows [T, ...]."""
    import torch
    G, T = layout.summary().num_groups, layout.total_tokens
    if padded.dim() < 2 or padded.shape[0] != G:
        raise ValueError(f"padded must be [G={G}, max_len, ...], got {tuple(padded.shape)}")
    L = padded.shape[1]
    tail = tuple(padded.shape[2:])
    if packed is None:
        packed = torch.empty((T,) + tail, dtype=padded.dtype, device="cuda")
    _check_tensor("packed", packed, (T,) + tail, padded.dtype)
    rb = _row_bytes(packed, 1)
    ptr = lambda t: ctypes.c_void_p(t.data_ptr() if t.numel() else None)
    check(load().pg_unpad_rows(layout.handle, ptr(padded), L, ctypes.c_int64(rb), ptr(packed),
                               _stream_handle(stream)), "pg_unpad_rows")
    return packed
