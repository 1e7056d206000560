"""Paged-KV grouped-query attention for AMD MI355X (gfx950).

A thin ctypes binding over ``libpa.so`` (C ABI in ``include/pa.h``).  It only
marshals arguments: it checks dtypes, devices and shapes of the torch tensors,
passes their device pointers and the current HIP stream, and raises
``PAError`` on a non-zero return code.  Every step of the computation runs in
the library's HIP kernels; there is no fallback path.  The first use of any
API name loads the library and raises ImportError if it has not been built
(``python -m prefill_block_table_amd.build``); the ``build`` submodule itself
imports without it.
"""
import importlib

_API = ("LIB_PATH", "PAError", "build_info", "decode", "decode_append", "decode_noalloc",
        "decode_workspace",
        "page_size_for_hybrid", "decode_input_prep", "prefill_workspace", "prefill_workspace_size",
        "prefill_varlen", "gemv",
        "decode_workspace_size", "kv_write", "kv_write_fused", "lib", "prefill_chunk",
        "slot_mapping", "strerror")

__all__ = list(_API)


def __getattr__(name):
    if name in _API:
        mod = importlib.import_module("._lib", __name__)
        return getattr(mod, name)
    raise AttributeError(f"module {__name__!r} has no attribute {name!r}")
