"""GPU: KV caches larger than 4 GiB with every referenced page placed past the
4 GiB byte offset, so each cache address needs more than 32 bits.  Where a
page sits does not enter the arithmetic, so the outputs (and the rows the
appending decode and the chunk write store) must equal, bit for bit, those of
the same case on its own small pool, which are checked against the oracle."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import bits, compare, log, to_dev

pytestmark = pytest.mark.gpu

NAN_BF16 = 0x7FC0


def _pa():
    import prefill_block_table_amd as pa
    return pa


def _base_page(small: np.ndarray) -> int:
    """First page id whose byte offset in a cache is above 2^32."""
    page_bytes = int(np.prod(small.shape[1:])) * 2
    return (1 << 32) // page_bytes + 1


def _big_pool(small: np.ndarray, base: int):
    """Device cache of base + P pages: NaN everywhere, the small pool at base..."""
    import torch
    big = torch.full((base + small.shape[0],) + small.shape[1:], NAN_BF16, dtype=torch.int16,
                     device="cuda").view(torch.bfloat16)
    big[base:] = to_dev(small)
    return big


def _release():
    import torch
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_decode_append_pages_above_4gib():
    import torch
    pa = _pa()
    c = W.decode_8k(seed=21)
    base = _base_page(c.k_cache)
    log(f"{c.name} pages at {base}.. (byte offset {base * c.k_cache[0].nbytes / 2**30:.2f} GiB)")
    q, sl = to_dev(c.q), to_dev(c.seq_lens)
    kn, vn = to_dev(c.k_new), to_dev(c.v_new)
    # small pool: the reference run
    k, v = to_dev(c.k_cache), to_dev(c.v_cache)
    bt = to_dev(c.block_tables)
    out_s = pa.decode_append(q, k, v, bt, sl, c.max_seq_len, c.scale, kn, vn)
    torch.cuda.synchronize()
    ref = oracle.decode(c.q, *oracle.kv_write(c.k_cache, c.v_cache, c.k_new, c.v_new,
                                              oracle.slot_mapping(c.positions, c.token_seq,
                                                                  c.block_tables, c.block_size)),
                        c.block_tables, c.seq_lens, c.block_size, c.scale)
    compare(bits(out_s), ref, c.name)
    k_small, v_small = bits(k), bits(v)
    del k, v
    # big pool, same pages shifted past 4 GiB
    kb, vb = _big_pool(c.k_cache, base), _big_pool(c.v_cache, base)
    btb = to_dev((c.block_tables.astype(np.int64) + base).astype(np.int32))
    slots = torch.full((1,), -7, dtype=torch.int64, device="cuda")
    out_b = pa.decode_append(q, kb, vb, btb, sl, c.max_seq_len, c.scale, kn, vn, slot_out=slots)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out_b), bits(out_s))
    expect_slot = oracle.slot_mapping(c.positions, c.token_seq, c.block_tables, c.block_size)[0]
    assert int(slots.item()) == int(expect_slot) + base * c.block_size
    assert np.array_equal(bits(kb[base:]), k_small) and np.array_equal(bits(vb[base:]), v_small)
    # the plain decode over the appended cache gives the same bits
    out_d = pa.decode(q, kb, vb, btb, sl, c.max_seq_len, c.scale)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out_d), bits(out_s))
    del kb, vb
    _release()


def test_prefill_chunk_pages_above_4gib():
    import torch
    pa = _pa()
    case = W.make_prefill_case("big_pool_prefill", 22, [(900, 1685)], 832, 6)
    ch = case.chunks[0]
    base = _base_page(case.k_cache)
    log(f"{case.name} q={ch.q_len}@{ch.start_pos} pages at {base}..")
    pos = to_dev(np.arange(ch.start_pos, ch.start_pos + ch.q_len, dtype=np.int64))
    q, kn, vn = to_dev(ch.q), to_dev(ch.k_new), to_dev(ch.v_new)
    k, v, bt = to_dev(case.k_cache), to_dev(case.v_cache), to_dev(case.block_table)
    pa.kv_write_fused(k, v, kn, vn, pos, bt)
    out_s = pa.prefill_chunk(q, k, v, bt, ch.start_pos, case.scale, causal=True)
    torch.cuda.synchronize()
    slots = oracle.slot_mapping(np.arange(ch.start_pos, ch.start_pos + ch.q_len, dtype=np.int64),
                                None, case.block_table, case.block_size)
    kr, vr = oracle.kv_write(case.k_cache, case.v_cache, ch.k_new, ch.v_new, slots)
    rows = np.linspace(0, ch.q_len - 1, 64).astype(np.int64)
    ref = oracle.prefill_chunk(ch.q, ch.start_pos, True, kr, vr, case.block_table,
                               case.block_size, case.scale, rows=rows)
    compare(bits(out_s)[rows], ref, case.name)
    k_small, v_small = bits(k), bits(v)
    del k, v
    kb, vb = _big_pool(case.k_cache, base), _big_pool(case.v_cache, base)
    btb = to_dev((case.block_table.astype(np.int64) + base).astype(np.int32))
    pa.kv_write_fused(kb, vb, kn, vn, pos, btb)
    out_b = pa.prefill_chunk(q, kb, vb, btb, ch.start_pos, case.scale, causal=True)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out_b), bits(out_s))
    assert np.array_equal(bits(kb[base:]), k_small) and np.array_equal(bits(vb[base:]), v_small)
    del kb, vb
    _release()
