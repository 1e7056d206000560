"""GPU parity: chunked-prefill paged GQA attention against the fp64 oracle."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import bits, compare, log, to_dev

pytestmark = pytest.mark.gpu


def _pa():
    import prefill_block_table_amd as pa
    return pa


def _sync():
    import torch
    torch.cuda.synchronize()


def _write_chunk_oracle(k, v, case, ch):
    pos = np.arange(ch.start_pos, ch.start_pos + ch.q_len, dtype=np.int64)
    slots = oracle.slot_mapping(pos, None, case.block_table, case.block_size)
    return oracle.kv_write(k, v, ch.k_new, ch.v_new, slots)


def run_chunks_gpu(case: W.PrefillCase):
    """Write each chunk's K/V, then run its attention; returns per-chunk outputs."""
    pa = _pa()
    k, v = to_dev(case.k_cache), to_dev(case.v_cache)
    bt = to_dev(case.block_table)
    outs = []
    for ch in case.chunks:
        pos = np.arange(ch.start_pos, ch.start_pos + ch.q_len, dtype=np.int64)
        pa.kv_write_fused(k, v, to_dev(ch.k_new), to_dev(ch.v_new), to_dev(pos), bt)
        out = pa.prefill_chunk(to_dev(ch.q), k, v, bt, ch.start_pos, case.scale,
                               causal=case.causal)
        outs.append(out)
    _sync()
    return [bits(o) for o in outs]


def run_chunks_oracle(case: W.PrefillCase, rows=None):
    k, v = case.k_cache, case.v_cache
    refs = []
    for i, ch in enumerate(case.chunks):
        k, v = _write_chunk_oracle(k, v, case, ch)
        r = None if rows is None else rows[i]
        refs.append(oracle.prefill_chunk(ch.q, ch.start_pos, case.causal, k, v, case.block_table,
                                         case.block_size, case.scale, rows=r))
    return refs


SMALL = [
    # (block_size, [(start, q_len), ...])
    (832, [(0, 2)]),
    (832, [(0, 128)]),
    (832, [(0, 129), (129, 127)]),
    (784, [(700, 300)]),
    (784, [(5, 1), (6, 63)]),
    (1024, [(1000, 65)]),
    (64, [(0, 200), (200, 77)]),
    (16, [(33, 150)]),
    (100, [(250, 256)]),
]


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("idx", range(len(SMALL)))
def test_small_chunks_all_rows(idx, causal):
    B, chunks = SMALL[idx]
    total = chunks[-1][0] + chunks[-1][1]
    pages = -(-total // B)
    c = W.make_prefill_case(f"small{idx}_b{B}", 60 + idx, chunks, B, pages + 3, causal=causal)
    log(f"{c.name} chunks={chunks} causal={causal}")
    got = run_chunks_gpu(c)
    ref = run_chunks_oracle(c)
    for i, (g, r) in enumerate(zip(got, ref)):
        compare(g, r, f"{c.name}[{i}]")


def _sample_rows(q_len, rng, n=24):
    fixed = [0, 1, 31, 32, 127, 128, 129, q_len // 2, q_len - 129, q_len - 128, q_len - 2,
             q_len - 1]
    fixed = [r for r in fixed if 0 <= r < q_len]
    return np.unique(np.concatenate([fixed, rng.integers(0, q_len, n)])).astype(np.int64)


def test_prefill_8k_chunks_all_rows():
    """The q=4096 @ 4096 and q=1685 @ 8192 chunks at full size (page 832,
    128-page pool), every row of both chunks against the fp64 oracle.  A
    sampled-row comparison runs first as a fast pre-check (it names a bad
    row before the full oracle has finished)."""
    c = W.prefill_8k()
    log(c.name)
    got = run_chunks_gpu(c)
    rng = np.random.default_rng(123)
    rows = [_sample_rows(ch.q_len, rng) for ch in c.chunks]
    pre = run_chunks_oracle(c, rows=rows)
    for i, (g, r) in enumerate(zip(got, pre)):
        compare(g[rows[i]], r, f"{c.name}[{i}] sampled pre-check")
    ref = run_chunks_oracle(c)
    for i, (g, r) in enumerate(zip(got, ref)):
        assert g.shape[0] == r.shape[0] == c.chunks[i].q_len
        log(f"{c.name}[{i}]: comparing all {r.shape[0]} rows x {r.shape[1]} heads x {r.shape[2]} dims")
        compare(g, r, f"{c.name}[{i}] all rows")


def test_prefill_repeatable():
    c = W.make_prefill_case("repeat", 70, [(1000, 700)], 832, 6)
    log(c.name)
    a = run_chunks_gpu(c)
    b = run_chunks_gpu(c)
    assert np.array_equal(a[0], b[0])


def test_single_kv_head_shard():
    c = W.make_prefill_case("hkv1", 71, [(300, 260)], 832, 4, hkv=1, hq=6)
    log(c.name)
    got = run_chunks_gpu(c)
    ref = run_chunks_oracle(c)
    compare(got[0], ref[0], c.name)


@pytest.mark.parametrize("hkv", [2, 3, 8])
def test_kv_head_counts(hkv):
    """Other KV-head counts: the workgroup-to-item map groups the 6 query heads
    of each KV head on one XCD for any count."""
    c = W.make_prefill_case(f"hkv{hkv}", 80 + hkv, [(300, 260)], 832, 4, hkv=hkv, hq=6 * hkv)
    log(c.name)
    got = run_chunks_gpu(c)
    ref = run_chunks_oracle(c)
    compare(got[0], ref[0], c.name)


# Chunks whose items do not fill whole rounds of 256 workgroups: the items of
# the last round are cut along their key groups and combined by a second
# launch (q=128 @ 8192: 24 items, 10 parts each; q=1 @ 32767: 24 items of one
# row; q=300 @ 5000 on page 16: 72 items, 3 parts; q=1685 @ 8192 is covered by
# the 8K test above).  q=128 @ 0: 2 parts of one key group each, so under the
# causal mask rows 0..63 have no key in the second part (its partial for them
# has l = 0 and must get weight 0, not NaN).
SPLIT = [
    (832, 8192, 128),
    (784, 32767, 1),
    (16, 5000, 300),
    (1024, 2000, 640),
    (832, 0, 128),
]


@pytest.mark.parametrize("idx", range(len(SPLIT)))
def test_split_chunks_all_rows(idx):
    import prefill_block_table_amd as pa
    B, start, q_len = SPLIT[idx]
    assert pa.prefill_workspace_size(q_len, start, B) > 0, "expected a split plan"
    c = W.make_prefill_case(f"split{idx}_b{B}", 90 + idx, [(start, q_len)], B,
                            -(-(start + q_len) // B) + 3)
    log(f"{c.name} start={start} q_len={q_len}")
    got = run_chunks_gpu(c)
    ref = run_chunks_oracle(c)
    compare(got[0], ref[0], c.name)
    again = run_chunks_gpu(c)
    assert np.array_equal(got[0], again[0]), "split path not repeatable"


# Several sequences in one call (pa_prefill_varlen): mixed lengths, a
# sequence with no rows, page sizes 832 / 16 / 784, causal and not.
VARLEN = [
    (832, [(0, 1), (700, 300), (4000, 129), (2496, 64)]),
    (16, [(33, 150), (0, 20), (1000, 0), (500, 1)]),
    (784, [(0, 256), (5000, 2)]),
]


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("idx", range(len(VARLEN)))
def test_varlen_all_rows(idx, causal):
    B, seqs = VARLEN[idx]
    pages = sum(-(-(s0 + n) // B) for s0, n in seqs)
    c = W.make_varlen_prefill_case(f"varlen{idx}_b{B}", 80 + idx, seqs, B, pages + 4, causal=causal)
    log(f"{c.name} seqs={seqs} causal={causal}")
    _check_varlen(c, causal)


@pytest.mark.parametrize("i", range(8))
def test_varlen_random_shapes(i):
    """Seeded random batches: 1-6 sequences, each at a random start with 0-400
    rows, random page size and KV-head count, mostly causal."""
    rng = np.random.default_rng(9000 + i)
    B = int(rng.choice([1, 16, 64, 784, 832, 1024, int(rng.integers(2, 1200))]))
    hkv = int(rng.choice([1, 2, 3, 4]))
    seqs = [(int(rng.integers(0, 2001)), int(rng.integers(0, 401))) for _ in range(int(rng.integers(1, 7)))]
    seqs = [(max(s0, 1) if n == 0 else s0, n) for s0, n in seqs]     # every sequence holds a token
    if all(n == 0 for _, n in seqs):
        seqs[0] = (seqs[0][0], 1)
    causal = bool(rng.integers(0, 4))
    B_pages = sum(-(-(s0 + n) // B) for s0, n in seqs)
    c = W.make_varlen_prefill_case(f"varlen_rand{i}_b{B}_hkv{hkv}", 9500 + i, seqs, B, B_pages + 4,
                                   causal=causal, hkv=hkv, hq=6 * hkv)
    log(f"{c.name} seqs={seqs} causal={causal}")
    _check_varlen(c, causal)


def test_varlen_many_sequences():
    """100 sequences in one call (more than one 64-entry pass of the
    workgroup's sequence search): one long chunk among 99 short ones at random
    starts, page 64, causal; the grid follows the rows batched (slots
    total_q / 128 + 100) rather than 100 x the longest sequence's tiles."""
    rng = np.random.default_rng(4242)
    seqs = [(1000, 1500)] + [(int(rng.integers(0, 501)), int(rng.integers(1, 41))) for _ in range(99)]
    order = rng.permutation(len(seqs))
    seqs = [seqs[j] for j in order]
    B = 64
    pages = sum(-(-(s0 + n) // B) for s0, n in seqs)
    c = W.make_varlen_prefill_case("varlen_100seqs_b64", 4243, seqs, B, pages + 4, causal=True)
    log(f"{c.name} long sequence at index {int(np.argmax([n for _, n in seqs]))}, total rows "
        f"{sum(n for _, n in seqs)}")
    _check_varlen(c, True)


def _check_varlen(c, causal):
    pa = _pa()
    B = c.block_size
    k, v = to_dev(c.k_cache), to_dev(c.v_cache)
    bt = to_dev(c.block_tables)
    kh, vh = c.k_cache, c.v_cache
    for s, ch in enumerate(c.chunks):
        if ch.q_len == 0:
            continue
        pos = np.arange(ch.start_pos, ch.start_pos + ch.q_len, dtype=np.int64)
        seq = np.full(ch.q_len, s, dtype=np.int32)
        pa.kv_write_fused(k, v, to_dev(ch.k_new), to_dev(ch.v_new), to_dev(pos), bt, to_dev(seq))
        kh, vh = oracle.kv_write(kh, vh, ch.k_new, ch.v_new,
                                 oracle.slot_mapping(pos, None, c.block_tables[s], B))
    lens = [ch.q_len for ch in c.chunks]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    used = np.array([ch.start_pos + ch.q_len for ch in c.chunks], dtype=np.int32)
    q = np.concatenate([ch.q for ch in c.chunks])
    out = pa.prefill_varlen(to_dev(q), k, v, bt, to_dev(cu), to_dev(used), max(lens), int(used.max()),
                            c.scale, causal=causal)
    _sync()
    ref = oracle.prefill_varlen(q, cu, used, causal, kh, vh, c.block_tables, B, c.scale)
    compare(bits(out), ref, c.name)


RANDOM_CASES = 12


@pytest.mark.parametrize("i", range(RANDOM_CASES))
def test_random_shapes(i):
    """Seeded random chunks: page size, KV-head count, start 0-2500, one or two
    contiguous chunks of 1-700 rows, causal or not; every row checked."""
    rng = np.random.default_rng(7000 + i)
    B = int(rng.choice([1, 16, 64, 100, 784, 832, 1024, int(rng.integers(2, 1200))]))
    hkv = int(rng.choice([1, 2, 3, 4, 4]))
    start = int(rng.integers(0, 2501))
    n1 = int(rng.integers(1, 701))
    chunks = [(start, n1)]
    if rng.integers(0, 2):
        chunks.append((start + n1, int(rng.integers(1, 701))))
    causal = bool(rng.integers(0, 4))          # mostly causal
    end = chunks[-1][0] + chunks[-1][1]
    c = W.make_prefill_case(f"rand{i}_b{B}_hkv{hkv}", 8000 + i, chunks, B, -(-end // B) + 2,
                            causal=causal, hkv=hkv, hq=6 * hkv)
    log(f"{c.name} chunks={chunks} causal={causal}")
    got = run_chunks_gpu(c)
    ref = run_chunks_oracle(c)
    for j, (g, r) in enumerate(zip(got, ref)):
        compare(g, r, f"{c.name}[{j}]")


def test_varlen_short_keys_unwritten_and_long_keys_clamped():
    """pa_prefill_varlen edge rules: a sequence given fewer keys than rows is
    left unwritten (its rows keep the caller's poison), and a key count above
    max_seqlen_k is clamped to it (the rows then sit at the last q_len of the
    first max_seqlen_k positions); a normal sequence beside them is exact."""
    import torch
    pa = _pa()
    B = 64
    seqs = [(300, 200), (0, 10), (700, 100)]          # A, B (keys cut to 5 below), C (800 keys)
    pages = sum(-(-(s0 + n) // B) for s0, n in seqs)
    c = W.make_varlen_prefill_case("varlen_edges", 95, seqs, B, pages + 4, causal=True)
    k, v = to_dev(c.k_cache), to_dev(c.v_cache)
    bt = to_dev(c.block_tables)
    kh, vh = c.k_cache, c.v_cache
    for s, ch in enumerate(c.chunks):
        pos = np.arange(ch.start_pos, ch.start_pos + ch.q_len, dtype=np.int64)
        seq = np.full(ch.q_len, s, dtype=np.int32)
        pa.kv_write_fused(k, v, to_dev(ch.k_new), to_dev(ch.v_new), to_dev(pos), bt, to_dev(seq))
        kh, vh = oracle.kv_write(kh, vh, ch.k_new, ch.v_new,
                                 oracle.slot_mapping(pos, None, c.block_tables[s], B))
    cu = np.array([0, 200, 210, 310], dtype=np.int32)
    used = np.array([500, 5, 950], dtype=np.int32)       # B: 5 keys < 10 rows; C: 950 > 800
    q = np.concatenate([ch.q for ch in c.chunks])
    out = torch.full((310, 24, 256), 0x7FC0, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    log(f"{c.name} used={used.tolist()} max_seqlen_k=800")
    pa.prefill_varlen(to_dev(q), k, v, bt, to_dev(cu), to_dev(used), 200, 800, c.scale,
                      causal=True, out=out)
    _sync()
    got = bits(out)
    assert np.all(got[200:210] == 0x7FC0), "rows of a sequence with fewer keys than rows were written"
    ref_a = oracle.prefill_chunk(c.chunks[0].q, 300, True, kh, vh, c.block_tables[0], B, c.scale)
    ref_c = oracle.prefill_chunk(c.chunks[2].q, 700, True, kh, vh, c.block_tables[2], B, c.scale)
    compare(got[:200], ref_a, c.name + " A")
    compare(got[210:], ref_c, c.name + " C (clamped)")
