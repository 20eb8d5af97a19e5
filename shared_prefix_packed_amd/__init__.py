"""Packed shared-prefix causal attention for MI355X (gfx950).

The product is libpg.so (C ABI in include/pg.h): a host layout builder and
HIP kernels for position ids, RoPE and the attention forward. This package is
its Python binding; importing it loads nothing until a function is called.
"""
from .api import (  # noqa: F401
    Layout,
    pg_attn_bwd,
    pg_attn_decode,
    pg_attn_decode_noalloc,
    pg_attn_fwd,
    pg_build_layout,
    pg_build_layout_host,
    pg_layout_upload,
    pg_pack_rows,
    pg_pad_rows,
    pg_position_ids_padded,
    pg_position_ids,
    pg_rope,
    pg_unpack_rows,
    pg_unpad_rows,
)
from ._lib import PgError, load  # noqa: F401
