"""GPU parity: paged GQA decode against the fp64 oracle (max abs <= 2e-2,
mean abs <= 2e-3), plus bitwise properties that hold for any correct split-K
implementation with a fixed merge order."""
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


def run_gpu(case: W.DecodeCase, tables=None, k_cache=None, v_cache=None, ws=None):
    pa = _pa()
    k = to_dev(case.k_cache if k_cache is None else k_cache)
    v = to_dev(case.v_cache if v_cache is None else v_cache)
    bt = to_dev(case.block_tables if tables is None else tables)
    if len(case.positions):
        pa.kv_write_fused(k, v, to_dev(case.k_new), to_dev(case.v_new), to_dev(case.positions),
                          bt, to_dev(case.token_seq))
    out = pa.decode(to_dev(case.q), k, v, bt, to_dev(case.seq_lens), case.max_seq_len,
                    case.scale, workspace=ws)
    _sync()
    return bits(out)


def run_oracle(case: W.DecodeCase, seqs=None):
    k, v = case.k_cache, case.v_cache
    if len(case.positions):
        slots = oracle.slot_mapping(case.positions, case.token_seq, case.block_tables,
                                    case.block_size)
        k, v = oracle.kv_write(k, v, case.k_new, case.v_new, slots)
    return oracle.decode(case.q, k, v, case.block_tables, case.seq_lens, case.block_size,
                         case.scale, seqs=seqs)


def test_tiny_decode():
    c = W.tiny_decode()
    log(c.name)
    compare(run_gpu(c), run_oracle(c), c.name)


def test_decode_8k_with_slot_mapping_write():
    c = W.decode_8k()
    log(c.name)
    compare(run_gpu(c), run_oracle(c), c.name)


@pytest.mark.parametrize("q_gain", [4.0, 16.0])
def test_peaked_attention_8k(q_gain):
    """q scaled by a power of two (exact in bf16), so the score spread grows
    to several times, then sixteen times, the workload's: each workgroup's
    partial is dominated by a few rows, the running max is re-based often,
    and the merge weighs partials whose maxima differ by hundreds (log2
    units).  The bf16 partials and the merge must stay within tolerance."""
    c = W.decode_8k(seed=12)
    c.q = W.f32_to_bf16_bits((oracle.bf16_bits_to_f64(c.q) * q_gain).astype(np.float32))
    log(f"{c.name} q x {q_gain}")
    compare(run_gpu(c), run_oracle(c), f"{c.name} q x {q_gain}")


@pytest.mark.parametrize("B", [784, 832, 1024])
def test_decode_32k_page_sweep(B):
    c = W.decode_32k(B)
    log(c.name)
    compare(run_gpu(c), run_oracle(c), c.name)


def test_batched_decode_16_seqs():
    c = W.batched_decode()
    log(c.name + " lens=" + ",".join(map(str, c.seq_lens.tolist())))
    compare(run_gpu(c), run_oracle(c), c.name)


@pytest.mark.parametrize("B", [784, 832, 1024, 64, 16, 1])
def test_ragged_boundary_lengths(B):
    """One batch whose sequences end on and around 64-token groups and pages."""
    lens = sorted({1, 2, 15, 16, 17, 63, 64, 65, 127, 129, B - 1, B, B + 1, 2 * B + 16,
                   3 * B - 1} - {0})
    lens = [n for n in lens if n >= 1 and n <= 4000]
    pages = sum(-(-n // B) for n in lens)
    c = W.make_decode_case(f"ragged_b{B}", 40 + B, lens, B, pages + 4, write_new_token=False)
    log(f"{c.name} lens={lens}")
    compare(run_gpu(c), run_oracle(c), c.name)


def test_one_token_context_returns_v_bitwise():
    c = W.make_decode_case("ctx1", 7, [1, 1, 1], 832, 6, write_new_token=False)
    log(c.name)
    got = run_gpu(c)
    for s in range(3):
        v0 = c.v_cache[c.block_tables[s, 0], 0]          # [4, 256]
        assert np.array_equal(got[s], np.repeat(v0, 6, axis=0))


def test_repeatable_and_page_permutation_invariant():
    """Same bits on a repeat run and after relabelling physical pages."""
    c = W.decode_32k(832, seed=44)
    log(c.name + " repeat / permutation")
    a = run_gpu(c)
    b = run_gpu(c)
    assert np.array_equal(a, b)
    rng = np.random.default_rng(9)
    perm = rng.permutation(c.num_pages)
    k2 = np.empty_like(c.k_cache)
    v2 = np.empty_like(c.v_cache)
    k2[perm] = c.k_cache
    v2[perm] = c.v_cache
    d = run_gpu(c, tables=perm[c.block_tables].astype(np.int32), k_cache=k2, v_cache=v2)
    assert np.array_equal(a, d)


def test_zero_length_sequence_gives_zeros_and_others_unaffected():
    c = W.make_decode_case("with_empty", 8, [300, 5, 900], 64, 40, write_new_token=False)
    c.seq_lens[1] = 0
    log(c.name)
    got = run_gpu(c)
    assert np.all(got[1] == 0)
    ref = run_oracle(c, seqs=[0, 2])
    compare(got[[0, 2]], ref[[0, 2]], c.name)


def test_single_kv_head_shard():
    """The per-GPU shape of a 4-way KV-head split: 1 KV head, 6 query heads."""
    c = W.make_decode_case("hkv1", 10, [5000, 1234], 832, 12, hkv=1, hq=6)
    log(c.name)
    compare(run_gpu(c), run_oracle(c), c.name)


def test_workspace_contents_never_read_uninitialised():
    """The workspace needs no initialisation: fill it with NaN bytes first."""
    import torch
    pa = _pa()
    for B, lens in ((64, [1, 2, 15, 17, 63, 65, 129, 191]), (832, [8193]), (16, [3, 4000, 70])):
        c = W.make_decode_case(f"ws_poison_b{B}", 90 + B, lens, B,
                               sum(-(-n // B) for n in lens) + 3, write_new_token=False)
        ws = pa.decode_workspace(len(lens), c.max_seq_len, B, device="cuda")
        ws.fill_(0xFF)                     # every float / int in it reads as NaN / -1
        log(f"{c.name} lens={lens}")
        compare(run_gpu(c, ws=ws), run_oracle(c), c.name)


def test_workspace_reuse_across_shapes():
    """A workspace sized for a large batch serves later, smaller calls."""
    pa = _pa()
    big = W.batched_decode(seed=50)
    small = W.decode_8k(seed=51)
    ws = pa.decode_workspace(16, big.max_seq_len, 832, device="cuda")
    log("workspace reuse")
    compare(run_gpu(big, ws=ws), run_oracle(big, seqs=range(16)), "reuse-big")
    compare(run_gpu(small, ws=ws), run_oracle(small), "reuse-small")
    compare(run_gpu(small, ws=ws), run_oracle(small), "reuse-small-again")


# ---------------------------------------------------------------------------
# pa_decode_append: the new token's KV write inside the decode launch.

def run_gpu_append(case: W.DecodeCase, ws=None):
    """Returns (out bits, k cache bits, v cache bits, slots) after one call."""
    import torch
    pa = _pa()
    S = case.q.shape[0]
    # the appended token of sequence s sits at position seq_lens[s] - 1
    assert np.array_equal(case.positions, case.seq_lens[case.token_seq].astype(np.int64) - 1)
    assert np.array_equal(case.token_seq, np.arange(S))
    k, v = to_dev(case.k_cache), to_dev(case.v_cache)
    slots = torch.full((S,), -7, dtype=torch.int64, device="cuda")
    out = pa.decode_append(to_dev(case.q), k, v, to_dev(case.block_tables), to_dev(case.seq_lens),
                           case.max_seq_len, case.scale, to_dev(case.k_new), to_dev(case.v_new),
                           workspace=ws, slot_out=slots)
    _sync()
    return bits(out), bits(k), bits(v), slots.cpu().numpy()


def _check_append(c: W.DecodeCase):
    got, kc, vc, slots = run_gpu_append(c)
    ref_slots = oracle.slot_mapping(c.positions, c.token_seq, c.block_tables, c.block_size)
    assert np.array_equal(slots, ref_slots)
    k_ref, v_ref = oracle.kv_write(c.k_cache, c.v_cache, c.k_new, c.v_new, ref_slots)
    assert np.array_equal(kc, k_ref) and np.array_equal(vc, v_ref)     # bit-exact cache
    compare(got, oracle.decode(c.q, k_ref, v_ref, c.block_tables, c.seq_lens, c.block_size,
                               c.scale), c.name + " append")
    # same bits as the two-launch path (kv_write_fused, then decode)
    assert np.array_equal(got, run_gpu(c))


def test_append_8k():
    c = W.decode_8k()
    log(c.name + " append")
    _check_append(c)


@pytest.mark.parametrize("B", [784, 1024])
def test_append_32k(B):
    """32767 cached tokens + the appended one (seq_len 32768)."""
    pages = -(-32768 // B)
    c = W.make_decode_case(f"append_ctx32768_b{B}", 70 + B, [32767], B, pages + 3)
    log(c.name)
    _check_append(c)


def test_append_batched_16_seqs():
    c = W.batched_decode()
    log(c.name + " append")
    _check_append(c)


@pytest.mark.parametrize("B", [832, 64, 16, 1])
def test_append_ragged_and_page_starts(B):
    """The appended token as the first row of a fresh page, the last row of a
    page, and mid-page, with NaN-poisoned unused rows."""
    lens = sorted({1, 2, 17, 64, 65, B, B + 1, 2 * B, 2 * B + 1, 3 * B - 1} - {0})
    lens = [n for n in lens if 1 <= n <= 4000]
    pages = sum(-(-(n + 1) // B) for n in lens)
    c = W.make_decode_case(f"append_ragged_b{B}", 60 + B, lens, B, pages + 4,
                           write_new_token=True)
    log(f"{c.name} lens={lens}")
    _check_append(c)


def test_append_single_kv_head_shard():
    c = W.make_decode_case("append_hkv1", 11, [4097, 833], 832, 12, hkv=1, hq=6)
    log(c.name)
    _check_append(c)


@pytest.mark.parametrize("hkv", [2, 3, 6, 8, 64])
def test_kv_head_counts(hkv):
    """KV-head counts the ABI takes besides 1 and 4: an item holds 4 KV heads
    when hkv % 4 == 0 (8 and 64: several items per sequence), 2 when
    hkv % 4 == 2 (two waves per head, each taking half of every step, merged
    through LDS), 1 otherwise (four waves per head); decode, the appending
    launch and the two-call path, with a one-token sequence among them."""
    lens = [2500, 517, 1] if hkv < 64 else [700, 33]
    B = 64
    pages = sum(-(-(n + 1) // B) for n in lens)
    c = W.make_decode_case(f"hkv{hkv}", 300 + hkv, lens, B, pages + 3, hkv=hkv, hq=6 * hkv)
    log(f"{c.name} lens={lens}")
    _check_append(c)


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 6, 7, 9, 12])
def test_steps_per_workgroup_sweep(n):
    """One sequence whose 16-token steps give every split workgroup n or n + 1
    steps, so the kernel's short path (all steps issued up front), its deep
    path with and without a steady round, and the round boundaries all run;
    both the two-call path and the appending launch."""
    L = 4096 * n + 1600            # cached tokens; +1 appended
    B = 832
    pages = -(-(L + 1) // B)
    c = W.make_decode_case(f"steps_per_wg_{n}", 300 + n, [L], B, pages + 3)
    log(c.name)
    _check_append(c)


@pytest.mark.parametrize("append", [False, True])
def test_more_than_256_sequences(append):
    """300 short sequences (1 to 700 tokens, page 64): the split kernel's scan
    over more sequences than one workgroup has threads, and items that start
    in one workgroup and end in another."""
    rng = np.random.Generator(np.random.PCG64(77))
    lens = [int(x) for x in rng.integers(1, 700, size=300)]
    B = 64
    pages = sum(-(-(n + 1) // B) for n in lens) + 3
    c = W.make_decode_case(f"seqs300_{'append' if append else 'decode'}", 78, lens, B, pages,
                           write_new_token=True)
    log(c.name)
    if append:
        _check_append(c)
    else:
        compare(run_gpu(c), run_oracle(c), c.name)


def test_many_sequences_with_long_ones():
    """300 sequences, most short, three of 12K-20K tokens: with more items
    than split workgroups the merge takes one workgroup per (head, sequence)
    over every slice, and the long items there combine dozens of partials."""
    rng = np.random.Generator(np.random.PCG64(79))
    lens = [int(x) for x in rng.integers(1, 400, size=300)]
    for j, n in ((5, 12000), (150, 20000), (299, 16001)):
        lens[j] = n
    B = 64
    pages = sum(-(-(n + 1) // B) for n in lens) + 3
    c = W.make_decode_case("seqs300_long", 80, lens, B, pages, write_new_token=True)
    log(c.name)
    _check_append(c)


RANDOM_CASES = 16


@pytest.mark.parametrize("i", range(RANDOM_CASES))
def test_random_shapes(i):
    """Seeded random shapes: page size (measured ones, odd ones, 1), KV-head
    count, 1-6 sequences of 1-6000 tokens, with or without the appended token."""
    rng = np.random.default_rng(5000 + i)
    B = int(rng.choice([1, 3, 16, 64, 100, 784, 832, 1024, int(rng.integers(2, 1200))]))
    hkv = int(rng.choice([1, 2, 3, 4, 4, 5, 6, 8]))
    S = int(rng.integers(1, 7))
    lens = [int(x) for x in rng.integers(1, 6001, size=S)]
    append = bool(rng.integers(0, 2))
    pages = sum(-(-(n + 1) // B) for n in lens) + 2
    c = W.make_decode_case(f"rand{i}_b{B}_hkv{hkv}", 6000 + i, lens, B, pages,
                           write_new_token=append, hkv=hkv, hq=6 * hkv)
    log(f"{c.name} lens={lens} append={append}")
    if append:
        _check_append(c)
    else:
        compare(run_gpu(c), run_oracle(c), c.name)


def test_seq_lens_clamped_to_range():
    """Lengths outside [0, max_seq_len] are clamped: a negative one gives an
    all-zero output, one above max_seq_len attends the first max_seq_len keys,
    and the other sequences are unaffected."""
    pa = _pa()
    c = W.make_decode_case("clamp", 41, [1, 2500, 700], 64, 4 + 40 + 11 + 3, write_new_token=False)
    ref = run_oracle(c)                     # lengths 1, 2500, 700
    lens = np.array([-5, 3000, 700], dtype=np.int32)
    log(f"{c.name} seq_lens={lens.tolist()} max_seq_len=2500")
    out = pa.decode(to_dev(c.q), to_dev(c.k_cache), to_dev(c.v_cache), to_dev(c.block_tables),
                    to_dev(lens), 2500, c.scale)
    _sync()
    got = bits(out)
    assert np.all(got[0] == 0)
    compare(got[1:], ref[1:], c.name)


@pytest.mark.parametrize("table_width", [47, 40])
def test_append_seq_lens_above_max_matches_two_call_path(table_width):
    """pa_decode_append with lengths outside [1, max_seq_len]: seq_lens
    [-5, 3000, 700] at max_seq_len 2500 on page 64.  The sequence above the
    bound attends its first 2500 cached keys unchanged and its new token goes
    to position 2999 (logical page 46), as pa_kv_write_fused at position
    seq_lens - 1 would put it: into the table's entry 46 when the row has 47
    entries, nowhere (slot -1) when it has 40.  Cache bits, output bits and
    the slots must equal the two-call path (kv_write_fused, then decode)."""
    import torch
    pa = _pa()
    B = 64
    c = W.make_decode_case(f"append_over_w{table_width}", 42, [1, 2500, 700], B, 4 + 40 + 11 + 3,
                           write_new_token=False, table_width=table_width)
    rng = np.random.Generator(np.random.PCG64(4242))
    k_new = W.normal_bf16(rng, (3, 4, 256))
    v_new = W.normal_bf16(rng, (3, 4, 256))
    lens = np.array([-5, 3000, 700], dtype=np.int32)
    bt = to_dev(c.block_tables)
    log(f"{c.name} seq_lens={lens.tolist()} max_seq_len=2500 bt_stride={c.block_tables.shape[1]}")
    # one launch
    k1, v1 = to_dev(c.k_cache), to_dev(c.v_cache)
    s1 = torch.full((3,), -7, dtype=torch.int64, device="cuda")
    o1 = pa.decode_append(to_dev(c.q), k1, v1, bt, to_dev(lens), 2500, c.scale, to_dev(k_new),
                          to_dev(v_new), slot_out=s1)
    # two calls
    k2, v2 = to_dev(c.k_cache), to_dev(c.v_cache)
    s2 = torch.full((3,), -7, dtype=torch.int64, device="cuda")
    pa.kv_write_fused(k2, v2, to_dev(k_new), to_dev(v_new), to_dev(lens.astype(np.int64) - 1), bt,
                      to_dev(np.arange(3, dtype=np.int32)), slot_out=s2)
    o2 = pa.decode(to_dev(c.q), k2, v2, bt, to_dev(lens), 2500, c.scale)
    _sync()
    assert np.array_equal(bits(k1), bits(k2)) and np.array_equal(bits(v1), bits(v2))
    assert np.array_equal(bits(o1), bits(o2))
    sl1, sl2 = s1.cpu().numpy(), s2.cpu().numpy()
    assert sl1[0] == -7                              # length <= 0: slot not written
    assert np.array_equal(sl1[1:], sl2[1:])
    want = -1 if table_width <= 46 else int(c.block_tables[1, 46]) * B + 2999 % B
    assert sl1[1] == want
    # the written row, and the outputs against the oracle (first 2500 keys)
    ref_slots = oracle.slot_mapping(np.array([2999, 699]), np.array([1, 2]), c.block_tables, B) \
        if table_width > 46 else oracle.slot_mapping(np.array([699]), np.array([2]), c.block_tables, B)
    kr, vr = oracle.kv_write(c.k_cache, c.v_cache, k_new[1:] if table_width > 46 else k_new[2:],
                             v_new[1:] if table_width > 46 else v_new[2:], ref_slots)
    assert np.array_equal(bits(k1), kr) and np.array_equal(bits(v1), vr)
    got = bits(o1)
    assert np.all(got[0] == 0)
    ref = oracle.decode(c.q, kr, vr, c.block_tables, np.array([1, 2500, 700], np.int32), B, c.scale,
                        seqs=[1, 2])
    compare(got[1:], ref[1:], c.name)


def _logical_case(L, seed):
    """Logical K/V rows [L, 4, 256] (bf16 bits), a query and a new token."""
    rng = np.random.Generator(np.random.PCG64(seed))
    K = W.normal_bf16(rng, (L, 4, 256))
    V = W.normal_bf16(rng, (L, 4, 256))
    q = W.normal_bf16(rng, (1, 24, 256))
    k_new = W.normal_bf16(rng, (1, 4, 256))
    v_new = W.normal_bf16(rng, (1, 4, 256))
    return K, V, q, k_new, v_new


def _paged(K, V, B, seed):
    """Lay logical rows out in pages of B rows, in a random physical order
    (pool of ceil(1.25 n) + 1 pages, the rest NaN); returns caches and the
    block-table row (one entry more than the rows need, for an appended row)."""
    L = K.shape[0]
    n = -(-(L + 1) // B)
    P = -(-5 * n // 4) + 1
    rng = np.random.Generator(np.random.PCG64(seed))
    perm = rng.permutation(P)[:n].astype(np.int32)
    kc = np.full((P, B, 4, 256), W.BF16_QNAN, np.uint16)
    vc = np.full((P, B, 4, 256), W.BF16_QNAN, np.uint16)
    for p in range(n):
        r = min(B, L - p * B)
        if r > 0:
            kc[perm[p], :r] = K[p * B:p * B + r]
            vc[perm[p], :r] = V[p * B:p * B + r]
    return kc, vc, perm[None, :]


@pytest.mark.parametrize("append", [False, True])
def test_page_size_bitwise_invariance(append):
    """The same logical K/V under pages of 784, 832 and 1024 tokens gives the
    same output bits (page-alignment post §9: page832 and page784 results can
    be bitwise identical).  Each of these page sizes is a whole number of the
    decode's 16-token steps (49, 52, 64), so the flattened step list, and with
    it every workgroup's keys and summation order, is the same.  32K decode,
    and the 8K appending decode (8192 cached keys + 1 written)."""
    pa = _pa()
    L = 8192 if append else 32768
    K, V, q, k_new, v_new = _logical_case(L, 31 + append)
    outs = {}
    for B in (784, 832, 1024):
        kc, vc, bt = _paged(K, V, B, 100 + B)
        k, v = to_dev(kc), to_dev(vc)
        n = L + 1 if append else L
        lens = np.array([n], np.int32)
        log(f"page-size invariance B={B} keys={n} append={append}")
        if append:
            out = pa.decode_append(to_dev(q), k, v, to_dev(bt), to_dev(lens), n, W.SCALE,
                                   to_dev(k_new), to_dev(v_new))
        else:
            out = pa.decode(to_dev(q), k, v, to_dev(bt), to_dev(lens), n, W.SCALE)
        _sync()
        outs[B] = bits(out)
        if append:
            # the appended row landed at logical position L
            kk = bits(k)
            assert np.array_equal(kk[bt[0, L // B], L % B], k_new[0])
    assert np.array_equal(outs[784], outs[832]), "784 vs 832 differ"
    assert np.array_equal(outs[1024], outs[832]), "1024 vs 832 differ"
    Kf = np.concatenate([K, k_new]) if append else K
    Vf = np.concatenate([V, v_new]) if append else V
    kc, vc, bt = _paged(Kf, Vf, 832, 7)
    ref = oracle.decode(q, kc, vc, bt, np.array([Kf.shape[0]], np.int32), 832, W.SCALE)
    compare(outs[832], ref, f"page-size invariance append={append}")
