"""ctypes loader and argument marshalling for libpa.so (see include/pa.h)."""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpa.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build the HIP library first with "
        "`python -m prefill_block_table_amd.build` (or __graft_entry__.build())")

lib = ctypes.CDLL(LIB_PATH)

_i32, _i64, _f32, _sz, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p

lib.pa_slot_mapping.argtypes = [_vp, _vp, _vp, _i32, _vp, _i32, _i32, _vp]
lib.pa_kv_write.argtypes = [_vp, _vp, _i64, _i32, _i32, _i32, _i32, _vp, _vp, _i32, _vp, _vp]
lib.pa_kv_write_fused.argtypes = [_vp, _vp, _i64, _i32, _i32, _i32, _i32, _vp, _vp, _i32,
                                  _vp, _vp, _vp, _i32, _vp, _vp]
lib.pa_decode_workspace_size.argtypes = [_i32, _i32, _i32, _i32, ctypes.POINTER(_sz)]
lib.pa_decode.argtypes = [_vp, _vp, _vp, _vp, _i64, _vp, _i32, _vp, _i32, _i32, _i32, _f32,
                          _i32, _i32, _i32, _vp, _sz, _vp]
lib.pa_decode_noalloc.argtypes = [_vp, _vp, _vp, _vp, _i64, _vp, _i32, _vp, _i32, _i32, _i32, _f32,
                                  _i32, _i32, _i32, _vp]
lib.pa_decode_append.argtypes = [_vp, _vp, _vp, _vp, _i64, _vp, _i32, _vp, _i32, _i32, _i32,
                                 _f32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _sz, _vp]
lib.pa_prefill_chunk.argtypes = [_vp, _vp, _i32, _i32, _i32, _vp, _vp, _i64, _vp, _i32, _i32,
                                 _f32, _i32, _i32, _i32, _vp, _sz, _vp]
lib.pa_prefill_varlen.argtypes = [_vp, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _i64,
                                  _vp, _i32, _i32, _f32, _i32, _i32, _i32, _vp]
lib.pa_prefill_varlen.restype = ctypes.c_int
lib.pa_prefill_workspace_size.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32, _i32, ctypes.POINTER(_sz)]
for _f in ("pa_slot_mapping", "pa_kv_write", "pa_kv_write_fused", "pa_decode_workspace_size",
           "pa_decode", "pa_decode_noalloc", "pa_decode_append", "pa_prefill_chunk", "pa_prefill_workspace_size"):
    getattr(lib, _f).restype = ctypes.c_int
lib.pa_decode_input_prep.argtypes = [_vp, _i64, _vp, _vp, _i32, _i64, _i64, _vp, _i32, _vp, _i32,
                                     _vp, _i32, _vp, _i32, _vp, _vp, _vp, _vp]
lib.pa_decode_input_prep.restype = ctypes.c_int
lib.pa_page_size_for_hybrid.argtypes = [_i64, _i64, _i32, ctypes.POINTER(_i32)]
lib.pa_page_size_for_hybrid.restype = ctypes.c_int
lib.pa_gemv_bf16.argtypes = [_vp, _i32, _vp, _vp, _i32, _i32, _i64, _vp]
lib.pa_gemv_bf16.restype = ctypes.c_int
lib.pa_strerror.argtypes = [ctypes.c_int]
lib.pa_strerror.restype = ctypes.c_char_p
lib.pa_build_info.argtypes = []
lib.pa_build_info.restype = ctypes.c_char_p

HEAD_DIM = 256
GQA = 6


class PAError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {strerror(code)} (code {code})")


def strerror(code: int) -> str:
    return lib.pa_strerror(int(code)).decode()


def build_info() -> str:
    return lib.pa_build_info().decode()


def _check(rc: int, where: str) -> None:
    if rc != 0:
        raise PAError(rc, where)


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t: torch.Tensor, name: str, dtypes, device=None, contiguous=True):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)


def _cache_geometry(k_cache: torch.Tensor, v_cache: torch.Tensor):
    """(num_pages, block_size, num_kv_heads, page_stride) of [P, B, Hkv, 256] caches.

    Pages may be strided (e.g. K and V views of a joint [P, 2, B, Hkv, D]
    tensor); rows inside a page must be contiguous.
    """
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, n, _BF16, contiguous=False)
        if t.dim() != 4 or t.shape[3] != HEAD_DIM:
            raise ValueError(f"{n} must be [num_pages, block_size, num_kv_heads, 256]")
        P, B, H, D = t.shape
        if t.stride(3) != 1 or t.stride(2) != D or t.stride(1) != H * D:
            raise ValueError(f"{n}: rows inside a page must be contiguous")
    if k_cache.shape != v_cache.shape or k_cache.stride(0) != v_cache.stride(0):
        raise ValueError("k_cache and v_cache must have the same shape and page stride")
    P, B, H, _ = k_cache.shape
    return P, B, H, k_cache.stride(0)


def slot_mapping(positions: torch.Tensor, block_table: torch.Tensor, block_size: int,
                 token_seq: torch.Tensor = None, out: torch.Tensor = None) -> torch.Tensor:
    """slot[i] = block_table[seq_i][pos_i // B] * B + pos_i % B (int64)."""
    _need(positions, "positions", (torch.int64,))
    _need(block_table, "block_table", (torch.int32,), positions.device)
    if token_seq is not None:
        _need(token_seq, "token_seq", (torch.int32,), positions.device)
    bt = block_table if block_table.dim() == 2 else block_table.view(1, -1)
    if out is None:
        out = torch.empty_like(positions)
    _need(out, "out", (torch.int64,), positions.device)
    _check(lib.pa_slot_mapping(_ptr(out), _ptr(positions), _ptr(token_seq), positions.numel(),
                               _ptr(bt), bt.shape[1], int(block_size), _stream(positions)),
           "pa_slot_mapping")
    return out


def kv_write(k_cache, v_cache, k_new, v_new, slot_mapping: torch.Tensor) -> None:
    """Scatter k_new/v_new [T, Hkv, 256] to the cache rows named by slot_mapping."""
    P, B, H, stride = _cache_geometry(k_cache, v_cache)
    _need(k_new, "k_new", _BF16, k_cache.device)
    _need(v_new, "v_new", _BF16, k_cache.device)
    _need(slot_mapping, "slot_mapping", (torch.int64,), k_cache.device)
    T = slot_mapping.numel()
    if k_new.shape != (T, H, HEAD_DIM) or v_new.shape != (T, H, HEAD_DIM):
        raise ValueError("k_new/v_new must be [num_tokens, num_kv_heads, 256]")
    _check(lib.pa_kv_write(_ptr(k_cache), _ptr(v_cache), stride, P, B, H, HEAD_DIM,
                           _ptr(k_new), _ptr(v_new), T, _ptr(slot_mapping), _stream(k_cache)),
           "pa_kv_write")


def kv_write_fused(k_cache, v_cache, k_new, v_new, positions: torch.Tensor,
                   block_table: torch.Tensor, token_seq: torch.Tensor = None,
                   slot_out: torch.Tensor = None) -> None:
    """Slot mapping and KV write in one launch; optionally stores the slots."""
    P, B, H, stride = _cache_geometry(k_cache, v_cache)
    _need(k_new, "k_new", _BF16, k_cache.device)
    _need(v_new, "v_new", _BF16, k_cache.device)
    _need(positions, "positions", (torch.int64,), k_cache.device)
    _need(block_table, "block_table", (torch.int32,), k_cache.device)
    if token_seq is not None:
        _need(token_seq, "token_seq", (torch.int32,), k_cache.device)
    if slot_out is not None:
        _need(slot_out, "slot_out", (torch.int64,), k_cache.device)
    bt = block_table if block_table.dim() == 2 else block_table.view(1, -1)
    T = positions.numel()
    if k_new.shape != (T, H, HEAD_DIM) or v_new.shape != (T, H, HEAD_DIM):
        raise ValueError("k_new/v_new must be [num_tokens, num_kv_heads, 256]")
    _check(lib.pa_kv_write_fused(_ptr(k_cache), _ptr(v_cache), stride, P, B, H, HEAD_DIM,
                                 _ptr(k_new), _ptr(v_new), T, _ptr(positions), _ptr(token_seq),
                                 _ptr(bt), bt.shape[1], _ptr(slot_out), _stream(k_cache)),
           "pa_kv_write_fused")


def decode_workspace_size(num_seqs: int, max_seq_len: int, block_size: int,
                          num_kv_heads: int = 4) -> int:
    n = ctypes.c_size_t(0)
    _check(lib.pa_decode_workspace_size(int(num_seqs), int(max_seq_len), int(block_size),
                                        int(num_kv_heads), ctypes.byref(n)),
           "pa_decode_workspace_size")
    return n.value


def decode_input_prep(sampled_token_ids, position: int, input_ids, positions, query_start_loc,
                      seq_lens, discard_request_mask, block_sizes=None, block_table_ptrs=None,
                      slot_mapping_ptrs=None, mrope: bool = False, mrope_delta: int = 0,
                      is_token_ids=None):
    """One launch that writes a single-token decode step's inputs and metadata
    (see pa_decode_input_prep in include/pa.h).

    sampled_token_ids int64 [>=1]; input_ids int32; positions int64 ([N] or,
    with mrope, [3, N]); query_start_loc, seq_lens int32; discard_request_mask
    and is_token_ids bool or uint8; block_sizes int32 [G]; block_table_ptrs and
    slot_mapping_ptrs uint64/int64 [G] holding device addresses (int32 rows,
    int64 outputs).  All on the device.  Enqueued on the current stream."""
    dev = input_ids.device
    _need(sampled_token_ids, "sampled_token_ids", (torch.int64,), dev)
    _need(input_ids, "input_ids", (torch.int32,), dev)
    _need(positions, "positions", (torch.int64,), dev)
    _need(query_start_loc, "query_start_loc", (torch.int32,), dev)
    _need(seq_lens, "seq_lens", (torch.int32,), dev)
    _need(discard_request_mask, "discard_request_mask", (torch.bool, torch.uint8), dev)
    if is_token_ids is not None:
        _need(is_token_ids, "is_token_ids", (torch.bool, torch.uint8), dev)
    stride = 0
    if mrope:
        if positions.dim() != 2 or positions.shape[0] != 3:
            raise ValueError("with mrope, positions must be [3, N]")
        stride = positions.stride(0)
    G = 0 if block_sizes is None else int(block_sizes.numel())
    if G:
        _need(block_sizes, "block_sizes", (torch.int32,), dev)
        _need(block_table_ptrs, "block_table_ptrs", (torch.uint64, torch.int64), dev)
        _need(slot_mapping_ptrs, "slot_mapping_ptrs", (torch.uint64, torch.int64), dev)
        if block_table_ptrs.numel() < G or slot_mapping_ptrs.numel() < G:
            raise ValueError("one block-table and one slot-mapping address per group")
    _check(lib.pa_decode_input_prep(
        _ptr(sampled_token_ids), int(position), _ptr(input_ids), _ptr(positions), int(bool(mrope)),
        int(stride), int(mrope_delta), _ptr(query_start_loc), int(query_start_loc.numel()),
        _ptr(seq_lens), int(seq_lens.numel()), _ptr(discard_request_mask),
        int(discard_request_mask.numel()), _ptr(is_token_ids) if is_token_ids is not None else None,
        G, _ptr(block_sizes) if G else None, _ptr(block_table_ptrs) if G else None,
        _ptr(slot_mapping_ptrs) if G else None, _stream(input_ids)), "pa_decode_input_prep")


def page_size_for_hybrid(mamba_page_bytes: int, attn_page_bytes_per_token: int = 4096,
                         alignment_tokens: int = 64) -> int:
    """KV page size in tokens for a hybrid attention / Mamba model (see
    pa_page_size_for_hybrid in include/pa.h)."""
    out = ctypes.c_int32(0)
    _check(lib.pa_page_size_for_hybrid(int(mamba_page_bytes), int(attn_page_bytes_per_token),
                                       int(alignment_tokens), ctypes.byref(out)),
           "pa_page_size_for_hybrid")
    return out.value


def gemv(W: torch.Tensor, x: torch.Tensor, out: torch.Tensor = None,
         out_dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
    """y = W x for bf16 W [N, K] (row stride ldw = W.stride(0)) and bf16 x [K];
    y is bf16 or float32 [N] (see pa_gemv_bf16 in include/pa.h)."""
    _need(W, "W", _BF16, contiguous=False)
    _need(x, "x", _BF16, device=W.device)
    if W.dim() != 2 or W.stride(1) != 1:
        raise ValueError("W must be [N, K] with unit stride along K")
    N, K = W.shape
    if x.dim() != 1 or x.shape[0] != K:
        raise ValueError("x must be [K]")
    if out is None:
        out = torch.empty(N, dtype=out_dtype, device=W.device)
    _need(out, "out", (torch.bfloat16, torch.float32), device=W.device)
    if out.shape != (N,):
        raise ValueError("out must be [N]")
    ldw = W.stride(0) if (N > 1 and K > 0) else K
    _check(lib.pa_gemv_bf16(_ptr(out), int(out.dtype == torch.float32), _ptr(W), _ptr(x), N, K,
                            ldw, _stream(W)), "pa_gemv_bf16")
    return out


def decode_workspace(num_seqs: int, max_seq_len: int, block_size: int, num_kv_heads: int = 4,
                     device="cuda") -> torch.Tensor:
    """A workspace of the size pa_decode needs (reusable; no initialisation needed)."""
    return torch.empty(decode_workspace_size(num_seqs, max_seq_len, block_size, num_kv_heads),
                       dtype=torch.uint8, device=device)


def decode(q, k_cache, v_cache, block_table, seq_lens, max_seq_len: int, scale: float,
           workspace: torch.Tensor = None, out: torch.Tensor = None) -> torch.Tensor:
    """q [S, 6*Hkv, 256] -> out [S, 6*Hkv, 256] bf16 (one query per sequence)."""
    P, B, H, stride = _cache_geometry(k_cache, v_cache)
    _need(q, "q", _BF16, k_cache.device)
    _need(block_table, "block_table", (torch.int32,), k_cache.device)
    _need(seq_lens, "seq_lens", (torch.int32,), k_cache.device)
    S = q.shape[0]
    if q.shape != (S, GQA * H, HEAD_DIM):
        raise ValueError("q must be [num_seqs, 6 * num_kv_heads, 256]")
    bt = block_table if block_table.dim() == 2 else block_table.view(1, -1)
    if bt.shape[0] < S or seq_lens.numel() < S:
        raise ValueError("block_table / seq_lens have fewer rows than q")
    if workspace is None:
        workspace = decode_workspace(S, max_seq_len, B, H, device=q.device)
    _need(workspace, "workspace", (torch.uint8,), k_cache.device)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", _BF16, k_cache.device)
    _check(lib.pa_decode(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), stride, _ptr(bt),
                         bt.shape[1], _ptr(seq_lens), S, int(max_seq_len), B, float(scale),
                         GQA * H, H, HEAD_DIM, _ptr(workspace), workspace.numel(), _stream(q)),
           "pa_decode")
    return out


def decode_noalloc(q, k_cache, v_cache, block_table, seq_lens, max_seq_len: int, scale: float,
                   out: torch.Tensor) -> torch.Tensor:
    """decode() with no workspace and no allocation (pa_decode_noalloc): the
    library's own per-GPU scratch buffer holds the partials.  `out` must be
    given (this call allocates nothing)."""
    P, B, H, stride = _cache_geometry(k_cache, v_cache)
    _need(q, "q", _BF16, k_cache.device)
    _need(block_table, "block_table", (torch.int32,), k_cache.device)
    _need(seq_lens, "seq_lens", (torch.int32,), k_cache.device)
    _need(out, "out", _BF16, k_cache.device)
    S = q.shape[0]
    if q.shape != (S, GQA * H, HEAD_DIM) or out.shape != q.shape:
        raise ValueError("q and out must be [num_seqs, 6 * num_kv_heads, 256]")
    bt = block_table if block_table.dim() == 2 else block_table.view(1, -1)
    if bt.shape[0] < S or seq_lens.numel() < S:
        raise ValueError("block_table / seq_lens have fewer rows than q")
    if torch.cuda.current_device() != q.device.index:
        raise ValueError("pa_decode_noalloc runs on the current device; q is on another one")
    _check(lib.pa_decode_noalloc(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), stride, _ptr(bt),
                                 bt.shape[1], _ptr(seq_lens), S, int(max_seq_len), B, float(scale),
                                 GQA * H, H, HEAD_DIM, _stream(q)), "pa_decode_noalloc")
    return out


def decode_append(q, k_cache, v_cache, block_table, seq_lens, max_seq_len: int, scale: float,
                  k_new, v_new, workspace: torch.Tensor = None, out: torch.Tensor = None,
                  slot_out: torch.Tensor = None) -> torch.Tensor:
    """One decode step that first appends k_new/v_new [S, Hkv, 256] at position
    seq_lens[s] - 1 of each sequence (same launch), then attends as decode()."""
    P, B, H, stride = _cache_geometry(k_cache, v_cache)
    _need(q, "q", _BF16, k_cache.device)
    S = q.shape[0]
    for t, n in ((k_new, "k_new"), (v_new, "v_new")):
        _need(t, n, _BF16, k_cache.device)
        if t.shape != (S, H, HEAD_DIM):
            raise ValueError(f"{n} must be [num_seqs, num_kv_heads, 256]")
    _need(block_table, "block_table", (torch.int32,), k_cache.device)
    _need(seq_lens, "seq_lens", (torch.int32,), k_cache.device)
    if q.shape != (S, GQA * H, HEAD_DIM):
        raise ValueError("q must be [num_seqs, 6 * num_kv_heads, 256]")
    bt = block_table if block_table.dim() == 2 else block_table.view(1, -1)
    if bt.shape[0] < S or seq_lens.numel() < S:
        raise ValueError("block_table / seq_lens have fewer rows than q")
    if slot_out is not None:
        _need(slot_out, "slot_out", (torch.int64,), k_cache.device)
        if slot_out.numel() < S:
            raise ValueError("slot_out has fewer entries than q has sequences")
    if workspace is None:
        workspace = decode_workspace(S, max_seq_len, B, H, device=q.device)
    _need(workspace, "workspace", (torch.uint8,), k_cache.device)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", _BF16, k_cache.device)
    _check(lib.pa_decode_append(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), stride,
                                _ptr(bt), bt.shape[1], _ptr(seq_lens), S, int(max_seq_len), B,
                                float(scale), GQA * H, H, HEAD_DIM, _ptr(k_new), _ptr(v_new),
                                _ptr(slot_out), _ptr(workspace), workspace.numel(), _stream(q)),
           "pa_decode_append")
    return out


def prefill_varlen(q, k_cache, v_cache, block_table, cu_seqlens_q, seqused_k, max_seqlen_q: int,
                   max_seqlen_k: int, scale: float, causal: bool = True,
                   out: torch.Tensor = None) -> torch.Tensor:
    """Several sequences: q [total_q, 6*Hkv, 256]; sequence s owns rows
    cu_seqlens_q[s]..cu_seqlens_q[s+1]-1 and sees seqused_k[s] keys through
    block_table[s] (see pa_prefill_varlen in include/pa.h)."""
    P, B, H, stride = _cache_geometry(k_cache, v_cache)
    _need(q, "q", _BF16, k_cache.device)
    _need(block_table, "block_table", (torch.int32,), k_cache.device)
    _need(cu_seqlens_q, "cu_seqlens_q", (torch.int32,), k_cache.device)
    _need(seqused_k, "seqused_k", (torch.int32,), k_cache.device)
    total_q = q.shape[0]
    if q.shape != (total_q, GQA * H, HEAD_DIM):
        raise ValueError("q must be [total_q, 6 * num_kv_heads, 256]")
    num_seqs = seqused_k.numel()
    if cu_seqlens_q.numel() != num_seqs + 1 or block_table.dim() != 2 or block_table.shape[0] < num_seqs:
        raise ValueError("cu_seqlens_q [S+1], seqused_k [S], block_table [>=S, stride]")
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", _BF16, k_cache.device)
    _check(lib.pa_prefill_varlen(_ptr(out), _ptr(q), total_q, _ptr(cu_seqlens_q), _ptr(seqused_k),
                                 num_seqs, int(max_seqlen_q), int(max_seqlen_k), int(bool(causal)),
                                 _ptr(k_cache), _ptr(v_cache), stride, _ptr(block_table),
                                 block_table.shape[1], B, float(scale), GQA * H, H, HEAD_DIM,
                                 _stream(q)), "pa_prefill_varlen")
    return out


def prefill_workspace_size(q_len: int, start_pos: int, block_size: int, causal: bool = True,
                           num_kv_heads: int = 4) -> int:
    n = ctypes.c_size_t(0)
    _check(lib.pa_prefill_workspace_size(int(q_len), int(start_pos), int(bool(causal)), int(block_size),
                                         GQA * int(num_kv_heads), int(num_kv_heads), HEAD_DIM,
                                         ctypes.byref(n)), "pa_prefill_workspace_size")
    return n.value


def prefill_workspace(q_len: int, start_pos: int, block_size: int, causal: bool = True,
                      num_kv_heads: int = 4, device="cuda"):
    """A workspace for pa_prefill_chunk of this chunk shape (None if it needs none)."""
    n = prefill_workspace_size(q_len, start_pos, block_size, causal, num_kv_heads)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def prefill_chunk(q_chunk, k_cache, v_cache, block_table, start_pos: int, scale: float,
                  causal: bool = True, out: torch.Tensor = None,
                  workspace: torch.Tensor = None) -> torch.Tensor:
    """q_chunk [q_len, 6*Hkv, 256] at positions start_pos.. -> out, same shape (bf16).
    A workspace of the size prefill_workspace_size gives is allocated when none is passed."""
    P, B, H, stride = _cache_geometry(k_cache, v_cache)
    _need(q_chunk, "q_chunk", _BF16, k_cache.device)
    _need(block_table, "block_table", (torch.int32,), k_cache.device)
    q_len = q_chunk.shape[0]
    if q_chunk.shape != (q_len, GQA * H, HEAD_DIM):
        raise ValueError("q_chunk must be [q_len, 6 * num_kv_heads, 256]")
    bt = block_table.reshape(-1)
    if out is None:
        out = torch.empty_like(q_chunk)
    _need(out, "out", _BF16, k_cache.device)
    if workspace is None:
        workspace = prefill_workspace(q_len, start_pos, B, causal, H, device=k_cache.device)
    ws_ptr, ws_bytes = (None, 0) if workspace is None else (_ptr(workspace), workspace.numel() * workspace.element_size())
    _check(lib.pa_prefill_chunk(_ptr(out), _ptr(q_chunk), q_len, int(start_pos), int(bool(causal)),
                                _ptr(k_cache), _ptr(v_cache), stride, _ptr(bt), bt.numel(), B,
                                float(scale), GQA * H, H, HEAD_DIM, ws_ptr, ws_bytes, _stream(q_chunk)),
           "pa_prefill_chunk")
    return out
