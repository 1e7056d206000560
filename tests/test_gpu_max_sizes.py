"""GPU parity at the largest shapes the tests afford: one decode step with
the appended token at a 262144-token context (page 832; 16385 16-token steps,
64 per workgroup; the output and the whole written cache compared), and a 16384-row prefill chunk at page 784 (128 query tiles per
head: twelve full rounds of 256 workgroups), compared on rows sampled from every tile
class (first and last row of the chunk, tile and page edges, random rows)."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import bits, compare, log, to_dev

pytestmark = pytest.mark.gpu


def test_decode_append_262144_context():
    import test_gpu_decode as TD
    L, B = 262144, 832
    c = W.make_decode_case("decode_ctx262144_b832", 71, [L], B, -(-(L + 1) // B) + 3,
                           write_new_token=True)
    log(f"{c.name} seq_len={int(c.seq_lens[0])}")
    TD._check_append(c)


def test_prefill_16384_rows_sampled():
    import torch
    import prefill_block_table_amd as pa
    q_len, start, B = 16384, 0, 784
    c = W.make_prefill_case("prefill_q16384_b784", 72, [(start, q_len)], B, -(-q_len // B) + 2)
    ch = c.chunks[0]
    log(f"{c.name} q_len={q_len}")
    k, v, bt = to_dev(c.k_cache), to_dev(c.v_cache), to_dev(c.block_table)
    pos = np.arange(start, start + q_len, dtype=np.int64)
    pa.kv_write_fused(k, v, to_dev(ch.k_new), to_dev(ch.v_new), to_dev(pos), bt)
    out = pa.prefill_chunk(to_dev(ch.q), k, v, bt, start, c.scale, causal=True)
    torch.cuda.synchronize()
    got = bits(out)
    rng = np.random.default_rng(73)
    edges = {0, 1, 63, 64, 127, 128, 129, 783, 784, 785, 8191, 8192, q_len - 129, q_len - 128,
             q_len - 2, q_len - 1}
    rows = np.array(sorted(edges | set(int(x) for x in rng.integers(0, q_len, size=48))))
    slots = oracle.slot_mapping(pos, None, c.block_table, B)
    rk, rv = oracle.kv_write(c.k_cache, c.v_cache, ch.k_new, ch.v_new, slots)
    ref = oracle.prefill_chunk(ch.q, start, True, rk, rv, c.block_table, B, c.scale, rows=rows)
    compare(got[rows], ref, f"{c.name} ({len(rows)} rows)")
    assert np.all(np.isfinite(oracle.bf16_bits_to_f64(got))), "non-finite rows"


def test_decode_4000_short_sequences():
    """4000 sequences of 1-40 tokens (page 16), with the appended token: far
    more items than workgroups, most of them whole inside one workgroup."""
    import test_gpu_decode as TD
    rng = np.random.default_rng(74)
    lens = [int(x) for x in rng.integers(1, 41, size=4000)]
    B = 16
    c = W.make_decode_case("decode_4000_seqs_b16", 75, lens, B, sum(-(-(n + 1) // B) for n in lens) + 2,
                           write_new_token=True)
    log(f"{c.name} total tokens {sum(lens)}")
    TD._check_append(c)
