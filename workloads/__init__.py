"""Seeded synthetic inputs for paged-KV GQA attention.

This module is the only code shared by the fp64 oracle (``oracle/``) and the
HIP path (``prefill_block_table_amd``).  It draws random numbers and lays them
out; it computes nothing the attention method computes (no slot arithmetic,
no scores, no softmax).  Every array it returns is a host NumPy array.

Shapes follow the full-attention layer described in the page-alignment post
(luanjiahao.me, post on moving the KV page from 784 to 832 tokens), §4
"Actual Page Shape of Qwen3.5": 24 query heads, 4 KV heads, head size 256,
BF16, and a per-tensor cache of shape [num_pages, block_size, 4, 256].

Generator: ``numpy.random.Generator(PCG64(seed))``.  Draw order for every
configuration: block-table permutation, K pool, V pool, q, k_new, v_new.
Values are N(0, 1) drawn in float32 and rounded to bf16 (round to nearest,
ties to even).  Pages that no block table references, and cache rows past the
end of the context, are filled with ``fill_bits`` (a quiet NaN by default) so
that any read of them by mistake shows up in the output.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import numpy as np

NUM_Q_HEADS = 24
NUM_KV_HEADS = 4
HEAD_DIM = 256
SCALE = 1.0 / math.sqrt(HEAD_DIM)  # 0.0625, exact in fp32 and bf16

BF16_QNAN = 0x7FC0  # quiet NaN bit pattern


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits.

    Inputs here are finite normal draws, so no NaN/Inf special-casing is needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    return f32_to_bf16_bits(rng.standard_normal(size=shape, dtype=np.float32))


@dataclasses.dataclass
class DecodeCase:
    """A batch of single-token decodes, with the new token's K/V to write first.

    ``positions[i]`` is the position of the token written by write i, in
    sequence ``token_seq[i]``; ``seq_lens[s]`` counts the keys decode attends
    for sequence s (it already includes that token).
    """
    name: str
    block_size: int
    num_pages: int
    k_cache: np.ndarray      # uint16 [P, B, Hkv, D] (bf16 bits), before the write
    v_cache: np.ndarray
    block_tables: np.ndarray  # int32 [S, max_pages]
    seq_lens: np.ndarray     # int32 [S]
    q: np.ndarray            # uint16 [S, Hq, D]
    positions: np.ndarray    # int64 [T]
    token_seq: np.ndarray    # int32 [T]
    k_new: np.ndarray        # uint16 [T, Hkv, D]
    v_new: np.ndarray
    scale: float = SCALE

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max())


@dataclasses.dataclass
class PrefillChunk:
    q_len: int
    start_pos: int
    q: np.ndarray        # uint16 [q_len, Hq, D]
    k_new: np.ndarray    # uint16 [q_len, Hkv, D]  (written at start_pos..start_pos+q_len-1)
    v_new: np.ndarray


@dataclasses.dataclass
class PrefillCase:
    """One sequence prefilled in chunks; the cache holds tokens [0, first start)."""
    name: str
    block_size: int
    num_pages: int
    k_cache: np.ndarray
    v_cache: np.ndarray
    block_table: np.ndarray   # int32 [max_pages]
    chunks: List[PrefillChunk]
    causal: bool = True
    scale: float = SCALE


def _pages_for(n_tokens: int, block_size: int) -> int:
    return -(-n_tokens // block_size)


def _fill_pool(rng, num_pages, block_size, tables, lens, hkv, d, fill_bits):
    """Pool with N(0,1) rows for tokens [0, len) of every table, fill elsewhere.

    Rows are drawn page by page in increasing physical page order, so the draw
    is independent of the traversal order of any kernel.
    """
    k = np.full((num_pages, block_size, hkv, d), fill_bits, dtype=np.uint16)
    v = np.full((num_pages, block_size, hkv, d), fill_bits, dtype=np.uint16)
    rows = {}  # physical page -> number of live rows
    for table, n in zip(tables, lens):
        for lp in range(_pages_for(n, block_size)):
            rows[int(table[lp])] = min(block_size, n - lp * block_size)
    order = sorted(rows)
    for phys in order:
        k[phys, : rows[phys]] = normal_bf16(rng, (rows[phys], hkv, d))
    for phys in order:
        v[phys, : rows[phys]] = normal_bf16(rng, (rows[phys], hkv, d))
    return k, v


def _tables(rng, num_pages, pages_per_seq, sentinel_page):
    """Disjoint random tables; unused entries point at a poisoned sentinel page."""
    need = int(sum(pages_per_seq))
    perm = rng.permutation(num_pages - 1)  # the last page is the sentinel
    assert need <= num_pages - 1
    width = max(pages_per_seq)
    bt = np.full((len(pages_per_seq), width), sentinel_page, dtype=np.int32)
    off = 0
    for s, n in enumerate(pages_per_seq):
        bt[s, :n] = perm[off: off + n]
        off += n
    return bt


def make_decode_case(name: str, seed: int, ctx_lens, block_size: int, num_pages: int,
                     write_new_token: bool = True, fill_bits: int = BF16_QNAN,
                     hkv: int = NUM_KV_HEADS, hq: int = NUM_Q_HEADS, d: int = HEAD_DIM,
                     table_width: Optional[int] = None) -> DecodeCase:
    """Decode case: sequence s holds ``ctx_lens[s]`` tokens in the cache.

    With ``write_new_token`` each sequence gets one more token at position
    ``ctx_lens[s]`` (seq_len = position + 1, the single-token decode metadata
    of the input-prep article, jsqmd.com/news/1214744, §2); its K/V are in
    ``k_new``/``v_new`` and its cache row still holds ``fill_bits``.
    The last pool page is a sentinel: never referenced for data, all fill.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    ctx_lens = [int(c) for c in ctx_lens]
    seq_lens = [c + (1 if write_new_token else 0) for c in ctx_lens]
    pages = [_pages_for(n, block_size) for n in seq_lens]
    sentinel = num_pages - 1
    bt = _tables(rng, num_pages, pages, sentinel)
    if table_width is not None and table_width > bt.shape[1]:
        bt = np.concatenate(
            [bt, np.full((bt.shape[0], table_width - bt.shape[1]), sentinel, np.int32)], 1)
    k, v = _fill_pool(rng, num_pages, block_size, bt, ctx_lens, hkv, d, fill_bits)
    S = len(ctx_lens)
    q = normal_bf16(rng, (S, hq, d))
    T = S if write_new_token else 0
    k_new = normal_bf16(rng, (T, hkv, d))
    v_new = normal_bf16(rng, (T, hkv, d))
    positions = np.asarray(ctx_lens[:T], dtype=np.int64)
    token_seq = np.arange(T, dtype=np.int32)
    return DecodeCase(name, block_size, num_pages, k, v, bt,
                      np.asarray(seq_lens, np.int32), q, positions, token_seq, k_new, v_new)


def make_prefill_case(name: str, seed: int, chunks, block_size: int, num_pages: int,
                      causal: bool = True, fill_bits: int = BF16_QNAN,
                      hkv: int = NUM_KV_HEADS, hq: int = NUM_Q_HEADS, d: int = HEAD_DIM
                      ) -> PrefillCase:
    """One sequence; ``chunks`` is a list of (start_pos, q_len), contiguous.

    The cache holds tokens [0, chunks[0].start) on entry; each chunk's own K/V
    is written (by the caller) before that chunk's attention runs.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    chunks = [(int(s), int(n)) for s, n in chunks]
    for (s0, n0), (s1, _) in zip(chunks, chunks[1:]):
        assert s0 + n0 == s1, "chunks must be contiguous"
    total = chunks[-1][0] + chunks[-1][1]
    n_pages = _pages_for(total, block_size)
    sentinel = num_pages - 1
    bt = _tables(rng, num_pages, [n_pages], sentinel)[0]
    k, v = _fill_pool(rng, num_pages, block_size, [bt], [chunks[0][0]], hkv, d, fill_bits)
    out = []
    for s0, n in chunks:
        out.append(PrefillChunk(n, s0, None, None, None))
    for c in out:
        c.q = normal_bf16(rng, (c.q_len, hq, d))
    for c in out:
        c.k_new = normal_bf16(rng, (c.q_len, hkv, d))
    for c in out:
        c.v_new = normal_bf16(rng, (c.q_len, hkv, d))
    return PrefillCase(name, block_size, num_pages, k, v, bt, out, causal)


# ---------------------------------------------------------------------------
# The five named workloads (sizes fixed by the pages' model shape and the
# chunked-prefill / long-context tiers they measure).
# ---------------------------------------------------------------------------

def tiny_decode(seed: int = 1, fill_bits: int = BF16_QNAN) -> DecodeCase:
    """1 seq, 2000 tokens, page 832 (3 pages, last partial), pool 8, q=1."""
    return make_decode_case("tiny_decode_ctx2000_b832", seed, [2000], 832, 8,
                            write_new_token=False, fill_bits=fill_bits)


def decode_8k(seed: int = 2, fill_bits: int = BF16_QNAN) -> DecodeCase:
    """1 seq, 8192 cached tokens + 1 written at position 8192, page 832, pool 64."""
    return make_decode_case("decode_ctx8192_b832", seed, [8192], 832, 64, fill_bits=fill_bits)


@dataclasses.dataclass
class VarlenPrefillCase:
    """Several sequences, one chunk each, in one call: sequence s holds tokens
    [0, start_s) in the cache and prefills q_len_s more (its K/V to write first)."""
    name: str
    block_size: int
    num_pages: int
    k_cache: np.ndarray
    v_cache: np.ndarray
    block_tables: np.ndarray  # int32 [S, max_pages]
    chunks: List[PrefillChunk]
    causal: bool = True
    scale: float = SCALE


def make_varlen_prefill_case(name: str, seed: int, seqs, block_size: int, num_pages: int,
                             causal: bool = True, fill_bits: int = BF16_QNAN,
                             hkv: int = NUM_KV_HEADS, hq: int = NUM_Q_HEADS,
                             d: int = HEAD_DIM) -> VarlenPrefillCase:
    """``seqs`` is a list of (start_pos, q_len), one chunk per sequence."""
    rng = np.random.Generator(np.random.PCG64(seed))
    seqs = [(int(s0), int(n)) for s0, n in seqs]
    pages = [_pages_for(s0 + n, block_size) for s0, n in seqs]
    sentinel = num_pages - 1
    bts = _tables(rng, num_pages, pages, sentinel)
    k, v = _fill_pool(rng, num_pages, block_size, list(bts), [s0 for s0, _ in seqs], hkv, d, fill_bits)
    chunks = [PrefillChunk(n, s0, None, None, None) for s0, n in seqs]
    for c in chunks:
        c.q = normal_bf16(rng, (c.q_len, hq, d))
    for c in chunks:
        c.k_new = normal_bf16(rng, (c.q_len, hkv, d))
    for c in chunks:
        c.v_new = normal_bf16(rng, (c.q_len, hkv, d))
    return VarlenPrefillCase(name, block_size, num_pages, k, v, bts, chunks, causal)


def prefill_8k(seed: int = 3, fill_bits: int = BF16_QNAN) -> PrefillCase:
    """Chunk q=4096 at start 4096, then q=1685 at start 8192; page 832, pool 128."""
    return make_prefill_case("prefill_q4096_s4096_then_q1685_b832", seed,
                             [(4096, 4096), (8192, 1685)], 832, 128, fill_bits=fill_bits)


def decode_32k(block_size: int, seed: int = 4, fill_bits: int = BF16_QNAN) -> DecodeCase:
    """1 seq, 32768 tokens, page 784/832/1024, pool = ceil(1.25 * pages) (+1 sentinel)."""
    pages = _pages_for(32768, block_size)
    pool = math.ceil(1.25 * pages) + 1
    return make_decode_case(f"decode_ctx32768_b{block_size}", seed, [32768], block_size, pool,
                            write_new_token=False, fill_bits=fill_bits)


def batched_decode(seed: int = 5, fill_bits: int = BF16_QNAN) -> DecodeCase:
    """16 seqs, ctx ~ U[4096, 32768], +1 written token each, page 832, pool 1024."""
    rng = np.random.Generator(np.random.PCG64(seed + 1000))
    ctx = rng.integers(4096, 32768, size=16, endpoint=True)
    return make_decode_case("decode_batch16_ctx4k_32k_b832", seed, ctx, 832, 1024,
                            fill_bits=fill_bits)


# Decode-time linear layers (long-context inference measurement post,
# luanjiahao.me 2026-07-17, §5): weight shapes N x K.
GEMV_SHAPES = ((14336, 5120), (16384, 5120), (34816, 5120))


def make_gemv_case(seed: int, N: int, K: int, w_std: float = 0.02):
    """(W [N, K], x [K]) as bf16 bit patterns: W ~ N(0, w_std^2), the scale of
    a trained projection's weights, and x ~ N(0, 1), a normalised activation;
    both drawn in float32 and rounded to bf16.  Draw order: W, then x."""
    rng = np.random.Generator(np.random.PCG64(seed))
    W = f32_to_bf16_bits(rng.standard_normal(size=(N, K), dtype=np.float32) * np.float32(w_std))
    x = normal_bf16(rng, (K,))
    return W, x
