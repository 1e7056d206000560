"""Plain fp64 definitions of the paged-attention hot path (test infrastructure only).

Notation: B = block_size (tokens per physical page), Hq query heads, Hkv KV
heads, D head size.  Caches are [num_pages, B, Hkv, D] arrays of bf16 bit
patterns (uint16).  Nothing here is blocked, fused or reordered beyond what
the definition itself states.
"""
from __future__ import annotations

import numpy as np


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact value of bf16 bit patterns: the bits are the top half of an fp32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x) -> np.ndarray:
    """Round fp64 values to bf16, nearest with ties to even (finite inputs).

    Done in exact integer arithmetic on the fp64 value: x = m * 2^e with the
    bf16 significand holding 8 bits.  Used only to report the bf16 rounding
    of the oracle's own results; parity compares against the unrounded fp64.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    flat_in = x.reshape(-1)
    flat_out = out.reshape(-1)
    for i, v in enumerate(flat_in):
        v = float(v)
        sign = 0x8000 if (v < 0 or (v == 0 and np.signbit(v))) else 0
        a = abs(v)
        if a == 0.0:
            flat_out[i] = sign
            continue
        m, e = np.frexp(a)  # a = m * 2^e, 0.5 <= m < 1
        e = int(e)
        # bf16 normal: exponent field 1..254, value in [2^-126, 2^128)
        if e - 1 < -126:  # subnormal: quantum 2^-133
            q = a / 2.0 ** -133
            n = int(np.floor(q))
            rem = q - n
            if rem > 0.5 or (rem == 0.5 and n % 2 == 1):
                n += 1
            flat_out[i] = sign | n  # n == 128 rolls into the smallest normal
            continue
        q = m * 256.0  # 8 significant bits: 128 <= q < 256
        n = int(np.floor(q))
        rem = q - n
        if rem > 0.5 or (rem == 0.5 and n % 2 == 1):
            n += 1
        if n == 256:
            n = 128
            e += 1
        exp_field = e - 1 + 127
        if exp_field >= 255:
            flat_out[i] = sign | 0x7F80
            continue
        flat_out[i] = sign | (exp_field << 7) | (n - 128)
    return out


def slot_mapping(positions, token_seq, block_tables, block_size: int) -> np.ndarray:
    """KV-cache slot of each written token.

    Input-prep article (jsqmd.com/news/1214744), §3.2 and §5: the logical
    block is position // block_size, the block number is the block table's
    entry for it, the offset is position % block_size, and the slot is
    block_number * block_size + offset.  ``token_seq[i]`` selects the table
    row of token i (all zero for a single sequence).
    """
    pos = np.asarray(positions, dtype=np.int64)
    seq = np.zeros_like(pos) if token_seq is None else np.asarray(token_seq, dtype=np.int64)
    bt = np.asarray(block_tables)
    if bt.ndim == 1:
        bt = bt[None, :]
    if np.any(pos < 0):
        raise ValueError("negative position")
    logical_block = pos // block_size
    offset = pos % block_size
    block_number = bt[seq, logical_block].astype(np.int64)
    return block_number * block_size + offset


def kv_write(k_cache, v_cache, k_new, v_new, slots):
    """Scatter new K/V rows to their slots; returns new cache arrays.

    A slot s addresses row s of the cache seen as [num_pages * B, Hkv, D]
    (slot // B is the physical page, slot % B the row in it).  Slots outside
    [0, num_pages * B) are skipped (the pages say nothing about them; padding
    slots such as -1 are thereby ignored).  Works on raw bf16 bits.
    """
    k = np.array(k_cache, copy=True)
    v = np.array(v_cache, copy=True)
    P, B = k.shape[0], k.shape[1]
    kf = k.reshape(P * B, *k.shape[2:])
    vf = v.reshape(P * B, *v.shape[2:])
    for i, s in enumerate(np.asarray(slots, dtype=np.int64)):
        if 0 <= s < P * B:
            kf[s] = k_new[i]
            vf[s] = v_new[i]
    return k, v


def gather_kv(cache, block_table_row, seq_len: int, block_size: int) -> np.ndarray:
    """Logical rows [0, seq_len) of one sequence, through its block table.

    Page-alignment post (luanjiahao.me), §1: logical_page = t // BLOCK_SIZE,
    page_offset = t % BLOCK_SIZE, physical_page = block_table[logical_page].
    Returns the raw cache entries, shape [seq_len, Hkv, D].
    """
    t = np.arange(seq_len, dtype=np.int64)
    logical_page = t // block_size
    page_offset = t % block_size
    physical_page = np.asarray(block_table_row)[logical_page].astype(np.int64)
    return np.asarray(cache)[physical_page, page_offset]


def attend(q, q_positions, K, V, scale: float, causal: bool = True,
           return_weights: bool = False):
    """softmax(scale * q K^T) V per query head, in float64.

    q: [R, Hq, D]; K, V: [L, Hkv, D] (contiguous logical order); query row r
    sits at absolute position q_positions[r].  Query head h reads KV head
    h // (Hq // Hkv) (consecutive query heads share a KV head; the pages give
    24 query heads over 4 KV heads, GQA ratio 6, page-alignment post §4).
    Allowed keys: j <= q_positions[r] when causal, all L keys otherwise.
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    R, Hq, D = q.shape
    L, Hkv, _ = K.shape
    if L < 1:
        raise ValueError("attention over an empty key set is undefined")
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    group = Hq // Hkv
    qpos = np.asarray(q_positions, dtype=np.int64).reshape(R)
    j = np.arange(L, dtype=np.int64)
    allowed = (j[None, :] <= qpos[:, None]) if causal else np.ones((R, L), dtype=bool)
    if not np.all(allowed.any(axis=1)):
        raise ValueError("a query row has no allowed key")
    out = np.empty((R, Hq, D), dtype=np.float64)
    weights = np.empty((R, Hq, L), dtype=np.float64) if return_weights else None
    for h in range(Hq):
        g = h // group
        s = scale * (q[:, h, :] @ K[:, g, :].T)          # [R, L]
        s = np.where(allowed, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        p = np.exp(s - m)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ V[:, g, :]
        if return_weights:
            weights[:, h, :] = p
    return (out, weights) if return_weights else out


def decode(q, k_cache, v_cache, block_tables, seq_lens, block_size: int, scale: float,
           seqs=None) -> np.ndarray:
    """Single-token decode for each sequence: one query at position seq_len - 1.

    seq_len counts the keys attended, the new token included (the decode
    metadata is seq_lens = position + 1, input-prep article §2).  The
    page-contiguous decode walks every page of the sequence and skips none
    (page-alignment post §7), so all seq_len keys are attended.
    ``seqs`` restricts the computation to some sequences (others are NaN).
    q: [S, Hq, D] bf16 bits; returns fp64 [S, Hq, D].
    """
    q = np.asarray(q)
    S = q.shape[0]
    out = np.full(q.shape, np.nan, dtype=np.float64)
    for s in (range(S) if seqs is None else seqs):
        L = int(seq_lens[s])
        K = bf16_bits_to_f64(gather_kv(k_cache, block_tables[s], L, block_size))
        V = bf16_bits_to_f64(gather_kv(v_cache, block_tables[s], L, block_size))
        out[s] = attend(bf16_bits_to_f64(q[s:s + 1]), [L - 1], K, V, scale, causal=True)[0]
    return out


def prefill_chunk(q_chunk, start_pos: int, causal: bool, k_cache, v_cache, block_table_row,
                  block_size: int, scale: float, rows=None, row_block: int = 256) -> np.ndarray:
    """Attention for a chunk of q_len queries at positions start_pos + i.

    The chunk's own K/V must already be in the cache, so the key set is the
    first start_pos + q_len logical tokens.  Causal: row i attends keys
    j <= start_pos + i (complete causal attention of a chunked prefill,
    page-alignment post §5-§6); non-causal: all start_pos + q_len keys.
    ``rows`` computes only those chunk rows (returned in that order);
    rows are processed ``row_block`` at a time only to bound memory.
    q_chunk: [q_len, Hq, D] bf16 bits; returns fp64.
    """
    q_chunk = np.asarray(q_chunk)
    q_len = q_chunk.shape[0]
    if q_len < 1 or start_pos < 0:
        raise ValueError("q_len must be >= 1 and start_pos >= 0")
    kv_len = start_pos + q_len
    K = bf16_bits_to_f64(gather_kv(k_cache, block_table_row, kv_len, block_size))
    V = bf16_bits_to_f64(gather_kv(v_cache, block_table_row, kv_len, block_size))
    rows = np.arange(q_len) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty((len(rows), q_chunk.shape[1], q_chunk.shape[2]), dtype=np.float64)
    for b0 in range(0, len(rows), row_block):
        r = rows[b0:b0 + row_block]
        # causal rows never need keys past their own position
        keys = int(start_pos + r.max() + 1) if causal else kv_len
        out[b0:b0 + len(r)] = attend(bf16_bits_to_f64(q_chunk[r]), start_pos + r,
                                     K[:keys], V[:keys], scale, causal=causal)
    return out


def prefill_varlen(q, cu_seqlens_q, seqused_k, causal: bool, k_cache, v_cache, block_tables,
                   block_size: int, scale: float) -> np.ndarray:
    """Several sequences in one call, the vendor interface's form
    (page-alignment post §6: cu_seqlens_q, seqused_k, block_table; the page
    uses it with one sequence): sequence s's rows cu[s]..cu[s+1]-1 are the last
    q_len_s of its seqused_k[s] tokens, i.e. a chunk at start_pos =
    seqused_k[s] - q_len_s.  Returns the rows of every sequence in order."""
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    used = np.asarray(seqused_k, dtype=np.int64)
    outs = []
    for s in range(len(used)):
        c0, c1 = int(cu[s]), int(cu[s + 1])
        if c1 <= c0:
            continue
        outs.append(prefill_chunk(np.asarray(q)[c0:c1], int(used[s]) - (c1 - c0), causal, k_cache,
                                  v_cache, np.asarray(block_tables)[s], block_size, scale))
    return np.concatenate(outs) if outs else np.zeros((0,) + np.shape(q)[1:])
