"""Seeded input generators: determinism, layout and poison placement (CPU only)."""
import numpy as np

import workloads as W


def test_bf16_rounding_of_inputs():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.0e-39], np.float32)
    assert [int(b) for b in W.f32_to_bf16_bits(x)] == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x0021]


def test_tiny_decode_layout_and_determinism():
    a = W.tiny_decode()
    b = W.tiny_decode()
    assert np.array_equal(a.k_cache, b.k_cache) and np.array_equal(a.q, b.q)
    assert a.block_tables.shape == (1, 3) and a.seq_lens.tolist() == [2000]
    assert len(set(a.block_tables[0].tolist())) == 3
    assert a.num_pages - 1 not in a.block_tables[0].tolist()    # sentinel unused
    last = a.block_tables[0, 2]
    live = 2000 - 2 * 832
    assert not np.any(a.k_cache[last, :live] == W.BF16_QNAN)
    assert np.all(a.k_cache[last, live:] == W.BF16_QNAN)       # past the context: poison
    assert np.all(a.v_cache[a.num_pages - 1] == W.BF16_QNAN)
    assert a.k_new.shape[0] == 0


def test_decode_8k_shapes():
    c = W.decode_8k()
    assert c.seq_lens.tolist() == [8193] and c.positions.tolist() == [8192]
    assert c.block_tables.shape == (1, 10)
    # the new token's row still holds poison until it is written
    page = c.block_tables[0, 8192 // 832]
    assert np.all(c.k_cache[page, 8192 % 832] == W.BF16_QNAN)
    assert int(c.seq_lens.sum()) * 4 * 256 * 2 * 2 == 33_558_528


def test_prefill_case_shapes():
    c = W.make_prefill_case("t", 9, [(100, 50), (150, 7)], 64, 8)
    assert [ch.q_len for ch in c.chunks] == [50, 7]
    assert c.chunks[0].q.shape == (50, 24, 256) and c.chunks[1].k_new.shape == (7, 4, 256)
    assert len(c.block_table) == 3
    assert np.all(c.k_cache[c.block_table[1], 100 - 64:] == W.BF16_QNAN)


def test_batched_decode_tables_disjoint():
    c = W.make_decode_case("b", 3, [70, 5, 129], 16, 40)
    used = []
    for s, L in enumerate(c.seq_lens):
        used += c.block_tables[s, : -(-int(L) // 16)].tolist()
    assert len(used) == len(set(used))
    assert c.seq_lens.tolist() == [71, 6, 130]
    assert c.token_seq.tolist() == [0, 1, 2]
