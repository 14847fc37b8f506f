"""xKV on AMD Instinct MI355X: cross-layer low-rank KV-cache compression and
Selective Reconstruction decode, behind the C ABI of libxkv.so (include/xkv.h).

The compute path is HIP only; this package marshals arguments.  Importing it
does not load the library; the first call does, and raises if it is missing.
"""
from ._lib import (  # noqa: F401
    XKV_BF16, XKV_F32, XkvError, Context, lib, LIB_PATH, make_desc, compress_ws_size, compress_sides,
    sr_args, sr_ws_size, sr_select, sr_attend, sr_decode, gram, topk, host_eigh,
    dense_args, dense_ws_size, dense_decode, rope_rows, rank_stats, rank_allocate, append_args, append_ws_size,
    compress_append,
)
from .xkv import compress, LayerDecoder, dtype_code  # noqa: F401
