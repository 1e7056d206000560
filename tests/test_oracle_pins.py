"""Pins of the fp64 oracle against things other than itself (CPU only).

Each test checks the oracle against what the pages or the mathematics fix:
the pages' printed page facts (tests/golden), exact bit patterns of the bf16
format, a pure-Python brute force over contiguous K/V, closed forms,
invariants, and PyTorch's scaled_dot_product_attention in float64 as an
independent library routine.  ``test_oracle_mutants.py`` plants plausible
mistakes in the oracle and checks that these pins catch them.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import paged_attention as pa
from workloads import f32_to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------
# helpers that build inputs without using the oracle's own index arithmetic
# ----------------------------------------------------------------------------

def _rand_bf16(rng, shape, scale=1.0):
    return f32_to_bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32))


def _page_out(contig, block_size, num_pages, table, fill=0x7FC0):
    """Place contiguous logical rows into a pool by walking the pages in order.

    Logical page p holds tokens p*B .. p*B+B-1; this walks (page, row) pairs
    with nested loops instead of the // and % of the oracle.
    """
    L = contig.shape[0]
    pool = np.full((num_pages, block_size) + contig.shape[1:], fill, dtype=np.uint16)
    t = 0
    p = 0
    while t < L:
        for r in range(block_size):
            if t >= L:
                break
            pool[table[p], r] = contig[t]
            t += 1
        p += 1
    return pool


def _brute_attention(q, qpos, K, V, scale, causal):
    """Pure-Python loops with math.exp over contiguous fp64 lists."""
    R, Hq, D = len(q), len(q[0]), len(q[0][0])
    L, Hkv = len(K), len(K[0])
    group = Hq // Hkv
    out = []
    for r in range(R):
        rows = []
        for h in range(Hq):
            g = h // group
            keys = [j for j in range(L) if (not causal) or j <= qpos[r]]
            s = []
            for j in keys:
                acc = 0.0
                for d in range(D):
                    acc += q[r][h][d] * K[j][g][d]
                s.append(scale * acc)
            m = max(s)
            e = [math.exp(x - m) for x in s]
            z = math.fsum(e)
            o = []
            for d in range(D):
                o.append(math.fsum(e[k] * V[keys[k]][g][d] for k in range(len(keys))) / z)
            rows.append(o)
        out.append(rows)
    return np.array(out)


def _to_f64(bits):
    # independent of the oracle's converter: build the fp32 via struct packing
    import struct
    b = np.asarray(bits, dtype=np.uint16)
    flat = [struct.unpack("<f", struct.pack("<I", int(x) << 16))[0] for x in b.reshape(-1)]
    return np.array(flat, dtype=np.float64).reshape(b.shape)


# ----------------------------------------------------------------------------
# bf16 format
# ----------------------------------------------------------------------------

def test_bf16_decode_known_patterns():
    # IEEE-754 binary32 upper halves: sign, 8 exponent bits, 7 fraction bits
    cases = {0x3F80: 1.0, 0xC000: -2.0, 0x3E80: 0.25, 0x4049: 3.140625,
             0x0000: 0.0, 0x8000: -0.0, 0x0001: 2.0 ** -133, 0x0080: 2.0 ** -126,
             0x7F7F: (2 - 2 ** -7) * 2.0 ** 127, 0x3F81: 1 + 2 ** -7}
    got = pa.bf16_bits_to_f64(np.array(list(cases), dtype=np.uint16))
    assert list(got) == list(cases.values())
    assert np.isinf(pa.bf16_bits_to_f64(np.array([0x7F80], np.uint16)))[0]
    assert np.isnan(pa.bf16_bits_to_f64(np.array([0x7FC0], np.uint16)))[0]


def test_bf16_round_nearest_even():
    ulp = 2.0 ** -7
    cases = [(1.0, 0x3F80), (1 + ulp / 2, 0x3F80),            # tie -> even (down)
             (1 + 3 * ulp / 2, 0x3F82),                         # tie -> even (up)
             (1 + ulp / 2 + 2 ** -30, 0x3F81),                  # above the tie
             (-1.5, 0xBFC0), (2.0 ** -133, 0x0001), (2.0 ** -134, 0x0000),
             (3 * 2.0 ** -134, 0x0002), (0.0, 0x0000), (2.0 ** 128, 0x7F80),
             ((2 - 2 ** -8) * 2.0 ** 127, 0x7F80), ((2 - 2 ** -7) * 2.0 ** 127, 0x7F7F)]
    got = pa.f64_to_bf16_bits(np.array([c[0] for c in cases]))
    assert [int(x) for x in got] == [c[1] for c in cases]


def test_bf16_round_trip_matches_input_generator():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(2000).astype(np.float32)
    gen = f32_to_bf16_bits(x)
    assert np.array_equal(pa.f64_to_bf16_bits(x.astype(np.float64)), gen)
    assert np.array_equal(pa.f64_to_bf16_bits(pa.bf16_bits_to_f64(gen)), gen)


# ----------------------------------------------------------------------------
# printed page facts
# ----------------------------------------------------------------------------

def test_page_facts_golden():
    g = json.load(open(os.path.join(GOLDEN, "page_facts.json")))
    for bs, exp in g["group_split"].items():
        assert oracle.groups_in_page(int(bs)) == (exp["full_groups"], exp["tail_tokens"])
    assert oracle.smallest_aligned_page(g["smallest_aligned_page"]["from"]) == \
        g["smallest_aligned_page"]["to"]
    for bs, exp in g["capacity_increase_vs_784_percent"].items():
        pct = 100.0 * (int(bs) / 784 - 1)
        assert abs(pct - exp["value"]) <= exp["printed_precision"]
    for bs, nbytes in g["page_bytes"].items():
        if bs.isdigit():
            assert oracle.page_bytes(int(bs)) == nbytes
    shape = g["model_shape"]
    assert shape["query_heads"] // shape["kv_heads"] == shape["gqa_ratio"]


def test_decode_metadata_golden():
    g = json.load(open(os.path.join(GOLDEN, "decode_metadata.json")))
    B = g["benchmark_block_size"]
    pos = g["benchmark_position"]
    bt = np.arange(4096, dtype=np.int32)[::-1].copy()   # any table
    slot = oracle.slot_mapping([pos], None, bt, B)[0]
    assert slot // B == bt[g["benchmark_logical_block"]]
    assert slot % B == g["benchmark_page_offset"]


# ----------------------------------------------------------------------------
# slot mapping and KV write
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("B", [1, 3, 16, 784, 832, 1024])
def test_slot_mapping_brute_force(B):
    rng = np.random.default_rng(B)
    S, pages = 3, 5
    num_pages = S * pages + 2
    perm = rng.permutation(num_pages)
    bt = perm[: S * pages].reshape(S, pages).astype(np.int32)
    # brute force: enumerate every (seq, logical page, row) and its slot by counting
    expected = {}
    for s in range(S):
        t = 0
        for p in range(pages):
            for r in range(B):
                expected[(s, t)] = int(bt[s, p]) * B + r
                t += 1
    keys = list(expected)
    idx = rng.choice(len(keys), size=min(200, len(keys)), replace=False)
    seqs = np.array([keys[i][0] for i in idx], np.int32)
    pos = np.array([keys[i][1] for i in idx], np.int64)
    got = oracle.slot_mapping(pos, seqs, bt, B)
    assert got.dtype == np.int64
    assert [int(x) for x in got] == [expected[keys[i]] for i in idx]
    # injective over disjoint tables
    all_pos = np.array([k[1] for k in keys], np.int64)
    all_seq = np.array([k[0] for k in keys], np.int32)
    all_slots = oracle.slot_mapping(all_pos, all_seq, bt, B)
    assert len(set(all_slots.tolist())) == len(keys)


def test_slot_mapping_large_positions_int64():
    # page index * block_size exceeds int32 when both are large
    B = 1024
    bt = np.array([[3_000_000]], np.int32)
    got = oracle.slot_mapping([5], None, bt, B)[0]
    assert got == 3_000_000 * 1024 + 5 and got > 2 ** 31


def test_kv_write_bytes():
    rng = np.random.default_rng(7)
    P, B, H, D = 6, 5, 4, 8
    k0 = np.full((P, B, H, D), 0x7FC0, np.uint16)
    v0 = np.full((P, B, H, D), 0xFFC0, np.uint16)
    T = 7
    kn = _rand_bf16(rng, (T, H, D))
    vn = _rand_bf16(rng, (T, H, D))
    slots = np.array([0, 29, 13, -1, 30, 7, 12], np.int64)   # -1 and 30 are out of range
    k1, v1 = oracle.kv_write(k0, v0, kn, vn, slots)
    touched = set()
    for i, s in enumerate(slots):
        if 0 <= s < P * B:
            page, row = divmod(int(s), B)
            assert np.array_equal(k1[page, row], kn[i])
            assert np.array_equal(v1[page, row], vn[i])
            touched.add((page, row))
    for page in range(P):
        for row in range(B):
            if (page, row) not in touched:
                assert np.all(k1[page, row] == 0x7FC0) and np.all(v1[page, row] == 0xFFC0)
    # inputs untouched
    assert np.all(k0 == 0x7FC0)


# ----------------------------------------------------------------------------
# attention: brute force on tiny inputs, through random paged layouts
# ----------------------------------------------------------------------------

SMALL_SHAPES = [(6, 1, 4), (12, 2, 8), (24, 4, 16)]


@pytest.mark.parametrize("B", [3, 5, 8, 16])
@pytest.mark.parametrize("shape", SMALL_SHAPES)
def test_decode_vs_brute_force(B, shape):
    Hq, Hkv, D = shape
    rng = np.random.default_rng(100 * B + Hq)
    lens = [1, 2, B, B + 1, 3 * B - 1, 41]
    S = len(lens)
    pages = [-(-n // B) for n in lens]
    num_pages = sum(pages) + 3
    perm = rng.permutation(num_pages)
    bt = np.full((S, max(pages)), num_pages - 1, np.int32)
    k_pool = np.full((num_pages, B, Hkv, D), 0x7FC0, np.uint16)
    v_pool = k_pool.copy()
    contig = []
    off = 0
    for s, n in enumerate(lens):
        bt[s, :pages[s]] = perm[off: off + pages[s]]
        off += pages[s]
        Kc = _rand_bf16(rng, (n, Hkv, D))
        Vc = _rand_bf16(rng, (n, Hkv, D))
        contig.append((Kc, Vc))
        kp = _page_out(Kc, B, num_pages, bt[s])
        vp = _page_out(Vc, B, num_pages, bt[s])
        for p in range(pages[s]):
            k_pool[bt[s, p]] = kp[bt[s, p]]
            v_pool[bt[s, p]] = vp[bt[s, p]]
    q = _rand_bf16(rng, (S, Hq, D), scale=2.0)
    scale = 1.0 / math.sqrt(D) * 1.7
    got = oracle.decode(q, k_pool, v_pool, bt, np.array(lens, np.int32), B, scale)
    for s, n in enumerate(lens):
        Kc, Vc = contig[s]
        ref = _brute_attention(_to_f64(q[s:s + 1]).tolist(), [n - 1], _to_f64(Kc).tolist(),
                               _to_f64(Vc).tolist(), scale, causal=True)[0]
        np.testing.assert_allclose(got[s], ref, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("B,start,q_len", [(4, 0, 9), (5, 7, 6), (8, 13, 1), (3, 0, 1)])
def test_prefill_vs_brute_force(B, start, q_len, causal):
    Hq, Hkv, D = 12, 2, 8
    rng = np.random.default_rng(B * 31 + start)
    kv_len = start + q_len
    pages = -(-kv_len // B)
    num_pages = pages + 4
    bt = rng.permutation(num_pages)[:pages].astype(np.int32)
    Kc = _rand_bf16(rng, (kv_len, Hkv, D))
    Vc = _rand_bf16(rng, (kv_len, Hkv, D))
    k_pool = _page_out(Kc, B, num_pages, bt)
    v_pool = _page_out(Vc, B, num_pages, bt)
    q = _rand_bf16(rng, (q_len, Hq, D), scale=1.5)
    scale = 0.3
    got = oracle.prefill_chunk(q, start, causal, k_pool, v_pool, bt, B, scale, row_block=4)
    ref = _brute_attention(_to_f64(q).tolist(), [start + i for i in range(q_len)],
                           _to_f64(Kc).tolist(), _to_f64(Vc).tolist(), scale, causal)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


def test_full_shape_vs_brute_force_tiny_context():
    # the real 24/4/256 shape, page 832, a 3-token context
    Hq, Hkv, D, B = 24, 4, 256, 832
    rng = np.random.default_rng(5)
    Kc = _rand_bf16(rng, (3, Hkv, D))
    Vc = _rand_bf16(rng, (3, Hkv, D))
    bt = np.array([2], np.int32)
    k_pool = _page_out(Kc, B, 4, bt)
    v_pool = _page_out(Vc, B, 4, bt)
    q = _rand_bf16(rng, (1, Hq, D))
    got = oracle.decode(q, k_pool, v_pool, bt[None], np.array([3], np.int32), B, 0.0625)
    ref = _brute_attention(_to_f64(q).tolist(), [2], _to_f64(Kc).tolist(),
                           _to_f64(Vc).tolist(), 0.0625, True)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)


# ----------------------------------------------------------------------------
# library routine: torch SDPA in float64 on CPU
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [True, False])
def test_prefill_vs_torch_sdpa(causal):
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F
    Hq, Hkv, D, B = 24, 4, 256, 832
    rng = np.random.default_rng(11)
    start, q_len = 900, 70
    kv_len = start + q_len
    pages = -(-kv_len // B)
    bt = rng.permutation(5)[:pages].astype(np.int32)
    Kc = _rand_bf16(rng, (kv_len, Hkv, D))
    Vc = _rand_bf16(rng, (kv_len, Hkv, D))
    k_pool = _page_out(Kc, B, 5, bt)
    v_pool = _page_out(Vc, B, 5, bt)
    q = _rand_bf16(rng, (q_len, Hq, D))
    got = oracle.prefill_chunk(q, start, causal, k_pool, v_pool, bt, B, 0.0625)
    tq = torch.from_numpy(_to_f64(q)).permute(1, 0, 2)[None]           # [1, Hq, R, D]
    tk = torch.from_numpy(_to_f64(Kc)).permute(1, 0, 2)[None]
    tv = torch.from_numpy(_to_f64(Vc)).permute(1, 0, 2)[None]
    tk = tk.repeat_interleave(Hq // Hkv, dim=1)
    tv = tv.repeat_interleave(Hq // Hkv, dim=1)
    i = torch.arange(q_len)[:, None] + start
    j = torch.arange(kv_len)[None, :]
    mask = (j <= i) if causal else torch.ones(q_len, kv_len, dtype=torch.bool)
    ref = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=0.0625)
    ref = ref[0].permute(1, 0, 2).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-12)


def test_decode_vs_torch_sdpa():
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F
    Hq, Hkv, D, B = 24, 4, 256, 784
    rng = np.random.default_rng(12)
    L = 2 * B + 17
    pages = -(-L // B)
    bt = rng.permutation(6)[:pages].astype(np.int32)
    Kc = _rand_bf16(rng, (L, Hkv, D))
    Vc = _rand_bf16(rng, (L, Hkv, D))
    k_pool = _page_out(Kc, B, 6, bt)
    v_pool = _page_out(Vc, B, 6, bt)
    q = _rand_bf16(rng, (1, Hq, D), scale=3.0)
    got = oracle.decode(q, k_pool, v_pool, bt[None], np.array([L], np.int32), B, 0.0625)
    tq = torch.from_numpy(_to_f64(q)).permute(1, 0, 2)[None]
    tk = torch.from_numpy(_to_f64(Kc)).permute(1, 0, 2)[None].repeat_interleave(6, dim=1)
    tv = torch.from_numpy(_to_f64(Vc)).permute(1, 0, 2)[None].repeat_interleave(6, dim=1)
    ref = F.scaled_dot_product_attention(tq, tk, tv, scale=0.0625)[0].permute(1, 0, 2).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-12)


# ----------------------------------------------------------------------------
# closed forms and invariants
# ----------------------------------------------------------------------------

def _case(rng, B, L, Hq=24, Hkv=4, D=256, num_pages=None):
    pages = -(-L // B)
    num_pages = num_pages or pages + 2
    bt = rng.permutation(num_pages)[:pages].astype(np.int32)
    Kc = _rand_bf16(rng, (L, Hkv, D))
    Vc = _rand_bf16(rng, (L, Hkv, D))
    return bt, Kc, Vc, _page_out(Kc, B, num_pages, bt), _page_out(Vc, B, num_pages, bt)


def test_one_token_context_returns_v_exactly():
    rng = np.random.default_rng(21)
    bt, Kc, Vc, kp, vp = _case(rng, 832, 1)
    q = _rand_bf16(rng, (1, 24, 256), scale=5.0)
    got = oracle.decode(q, kp, vp, bt[None], np.array([1], np.int32), 832, 0.0625)
    expect = np.repeat(_to_f64(Vc[0]), 6, axis=0)          # head h reads kv head h // 6
    assert np.array_equal(got[0], expect)


def test_zero_query_gives_prefix_mean():
    rng = np.random.default_rng(22)
    B, start, q_len = 64, 100, 37
    bt, Kc, Vc, kp, vp = _case(rng, B, start + q_len)
    q = np.zeros((q_len, 24, 256), np.uint16)
    Vf = _to_f64(Vc)
    got = oracle.prefill_chunk(q, start, True, kp, vp, bt, B, 0.0625)
    for i in [0, 1, q_len // 2, q_len - 1]:
        mean = Vf[: start + i + 1].mean(axis=0)        # keys 0..start+i
        np.testing.assert_allclose(got[i], np.repeat(mean, 6, axis=0), rtol=1e-12, atol=1e-14)
    got_nc = oracle.prefill_chunk(q, start, False, kp, vp, bt, B, 0.0625)
    np.testing.assert_allclose(got_nc[0], np.repeat(Vf.mean(axis=0), 6, axis=0),
                               rtol=1e-12, atol=1e-14)
    # decode: seq_len keys, the last being the decoded token itself
    L = start + q_len
    gd = oracle.decode(q[:1], kp, vp, bt[None], np.array([L], np.int32), B, 0.0625)
    np.testing.assert_allclose(gd[0], np.repeat(Vf.mean(axis=0), 6, axis=0),
                               rtol=1e-12, atol=1e-14)


def test_constant_v_and_equal_keys():
    rng = np.random.default_rng(23)
    B, L = 16, 70
    bt, Kc, Vc, kp, vp = _case(rng, B, L, Hq=12, Hkv=2, D=8)
    q = _rand_bf16(rng, (1, 12, 8), scale=4.0)
    vconst = np.full_like(vp, 0x4040)   # 3.0
    got = oracle.decode(q, kp, vconst, bt[None], np.array([L], np.int32), B, 0.5)
    np.testing.assert_allclose(got, 3.0, rtol=1e-14)
    kconst = np.full_like(kp, 0x3F80)   # all keys equal -> uniform weights
    got = oracle.decode(q, kconst, vp, bt[None], np.array([L], np.int32), B, 0.5)
    mean = _to_f64(Vc).mean(axis=0)
    np.testing.assert_allclose(got[0], np.repeat(mean, 6, axis=0), rtol=1e-12, atol=1e-14)


def test_softmax_weights_rows_sum_to_one():
    rng = np.random.default_rng(24)
    R, L = 9, 50
    q = rng.standard_normal((R, 24, 256)) * 3
    K = rng.standard_normal((L, 4, 256))
    V = rng.standard_normal((L, 4, 256))
    pos = np.arange(R) + L - R
    out, w = oracle.attend(q, pos, K, V, 0.0625, causal=True, return_weights=True)
    assert np.all(w >= 0)
    np.testing.assert_allclose(w.sum(axis=2), 1.0, rtol=0, atol=1e-12)
    for r in range(R):
        assert np.all(w[r, :, pos[r] + 1:] == 0)
        assert np.all(w[r, :, : pos[r] + 1] > 0)
    np.testing.assert_allclose(out, np.einsum("rhl,lhd->rhd", w,
                                              np.repeat(V, 6, axis=1)), rtol=1e-12, atol=1e-13)


def test_physical_page_permutation_invariance():
    rng = np.random.default_rng(25)
    B, L = 832, 2000
    bt, Kc, Vc, kp, vp = _case(rng, B, L, num_pages=8)
    q = _rand_bf16(rng, (1, 24, 256))
    a = oracle.decode(q, kp, vp, bt[None], np.array([L], np.int32), B, 0.0625)
    perm = rng.permutation(8)           # physical page p moves to perm[p]
    kp2 = np.empty_like(kp)
    vp2 = np.empty_like(vp)
    kp2[perm] = kp
    vp2[perm] = vp
    b = oracle.decode(q, kp2, vp2, perm[bt][None].astype(np.int32), np.array([L], np.int32),
                      B, 0.0625)
    assert np.array_equal(a, b)


def test_page_size_invariance():
    rng = np.random.default_rng(26)
    L = 2500
    Kc = _rand_bf16(rng, (L, 4, 256))
    Vc = _rand_bf16(rng, (L, 4, 256))
    q = _rand_bf16(rng, (1, 24, 256))
    outs = []
    for B in (784, 832, 1024):
        pages = -(-L // B)
        bt = rng.permutation(pages + 1)[:pages].astype(np.int32)
        kp = _page_out(Kc, B, pages + 1, bt)
        vp = _page_out(Vc, B, pages + 1, bt)
        outs.append(oracle.decode(q, kp, vp, bt[None], np.array([L], np.int32), B, 0.0625))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[1], outs[2])


def test_chunking_identity_and_decode_is_last_prefill_row():
    rng = np.random.default_rng(27)
    B = 48
    total = 300
    bt, Kc, Vc, kp, vp = _case(rng, B, total)
    q_all = _rand_bf16(rng, (total, 24, 256))
    full = oracle.prefill_chunk(q_all, 0, True, kp, vp, bt, B, 0.0625)
    start = 173
    part = oracle.prefill_chunk(q_all[start:], start, True, kp, vp, bt, B, 0.0625)
    np.testing.assert_allclose(part, full[start:], rtol=1e-12, atol=1e-14)
    dec = oracle.decode(q_all[total - 1:], kp, vp, bt[None], np.array([total], np.int32),
                        B, 0.0625)
    np.testing.assert_allclose(dec[0], full[-1], rtol=1e-12, atol=1e-14)


def test_gqa_equals_mha_with_repeated_kv():
    rng = np.random.default_rng(28)
    L, R = 60, 5
    q = rng.standard_normal((R, 24, 32))
    K = rng.standard_normal((L, 4, 32))
    V = rng.standard_normal((L, 4, 32))
    pos = np.arange(R) + 40
    a = oracle.attend(q, pos, K, V, 0.2)
    b = oracle.attend(q, pos, np.repeat(K, 6, axis=1), np.repeat(V, 6, axis=1), 0.2)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-14)
    # distinct kv heads really produce distinct outputs for the 4 head groups
    assert not np.allclose(a[:, 0], a[:, 6])


def test_oracle_rejects_empty():
    with pytest.raises(ValueError):
        oracle.attend(np.zeros((1, 24, 8)), [0], np.zeros((0, 4, 8)), np.zeros((0, 4, 8)), 1.0)
    with pytest.raises(ValueError):
        oracle.prefill_chunk(np.zeros((0, 24, 8), np.uint16), 0, True,
                             np.zeros((1, 4, 4, 8), np.uint16), np.zeros((1, 4, 4, 8), np.uint16),
                             np.array([0], np.int32), 4, 1.0)


# ---- page-size derivation (page-alignment post, section 3) -------------------

def _page_facts():
    return json.load(open(os.path.join(GOLDEN, "page_facts.json")))


def test_page_derivation_reproduces_printed_pages():
    """784 at the generic alignment, 832 at the backend's 64, for every Mamba
    page size the printed pair allows (section 3), with the section 4 shape."""
    g = _page_facts()["page_derivation"]
    per_tok = oracle.attn_page_bytes_per_token(4, 256, 2)
    assert per_tok == 4096
    lo, hi = 48 * 16 * per_tok, 49 * 16 * per_tok          # (3145728, 3211264]
    for m in (lo + 1, lo + 4096, (lo + hi) // 2, hi - 1, hi):
        assert oracle.required_page_tokens(m, per_tok, g["alignment_generic"]) == g["default_page_generic"]
        assert oracle.required_page_tokens(m, per_tok, g["alignment_backend"]) == g["page_backend"]
    # just outside the range the generic page moves off 784
    assert oracle.required_page_tokens(lo, per_tok, 16) == 768
    assert oracle.required_page_tokens(hi + 1, per_tok, 16) == 800


def test_page_derivation_brute_force():
    """The result is the smallest multiple of the alignment whose attention
    page holds at least one Mamba page: checked by scanning multiples."""
    rng = np.random.Generator(np.random.PCG64(11))
    for _ in range(300):
        per_tok = int(rng.integers(1, 9000))
        align = int(rng.choice([1, 3, 16, 64, 128]))
        m = int(rng.integers(1, 5_000_000))
        tokens = align
        while tokens * per_tok < m:
            tokens += align
        assert oracle.required_page_tokens(m, per_tok, align) == tokens


def test_page_derivation_rejects_nonpositive():
    for args in ((0, 4096, 64), (1000, 0, 64), (1000, 4096, 0), (-5, 4096, 64)):
        with pytest.raises(ValueError):
            oracle.required_page_tokens(*args)


# ---- single-token decode input preparation (input-prep post) -----------------

def _prep_case(position, block_sizes, n_tokens=64, n_reqs=16, mrope=False, seed=0):
    rng = np.random.Generator(np.random.PCG64(seed))
    tables = [rng.permutation(4096)[: -(-(position + 1) // B) + 3].astype(np.int32) for B in block_sizes]
    poison = -7
    bufs = dict(
        input_ids=np.full(n_tokens, poison, np.int32),
        positions=np.full((3, n_tokens + 1) if mrope else n_tokens, poison, np.int64),
        query_start_loc=np.full(n_reqs + 1, poison, np.int32),
        seq_lens=np.full(n_reqs, poison, np.int32),
        discard_request_mask=np.ones(n_reqs, np.uint8),
    )
    slots = [np.full(n_tokens, poison, np.int64) for _ in block_sizes]
    return tables, bufs, slots


def test_input_prep_printed_closed_forms():
    """The pages' closed forms (section 2) at their benchmark configuration
    (section 11: position 24576, two KV groups of page 16, 128 request slots)."""
    f = json.load(open(os.path.join(GOLDEN, "input_prep_facts.json")))["benchmark_config"]
    P = f["position"]
    tables, bufs, slots = _prep_case(P, f["block_sizes"], n_tokens=f["max_num_tokens"],
                                     n_reqs=f["max_num_reqs"], mrope=True)
    out = oracle.decode_input_prep(np.array([151_643], np.int64), P, block_sizes=f["block_sizes"],
                                   block_tables=tables, slot_mappings=slots, mrope=True, **bufs)
    assert out["input_ids"][0] == 151_643 and np.all(out["input_ids"][1:] == -7)
    assert np.all(out["positions"][:, 0] == P) and np.all(out["positions"][:, 1:] == -7)
    assert out["query_start_loc"].tolist() == [0] + [1] * f["max_num_reqs"]
    assert out["seq_lens"].tolist() == [P + 1] + [0] * (f["max_num_reqs"] - 1)
    assert not out["discard_request_mask"].any()
    for B, row, sm in zip(f["block_sizes"], tables, out["slot_mappings"]):
        # section 3.2 at P = 24576, B = 16: logical block 1536, offset 0
        assert sm[0] == int(row[1536]) * 16 and np.all(sm[1:] == -7)


def test_input_prep_slot_matches_gather():
    """Slot of each group = the cache row that a page-table walk reaches for
    the position (brute force over a flattened pool), for pages 16/784/832."""
    for seed, P in enumerate([0, 1, 783, 784, 831, 832, 8192, 24576, 32767]):
        Bs = [16, 784, 832]
        tables, bufs, slots = _prep_case(P, Bs, seed=seed)
        out = oracle.decode_input_prep(np.array([5], np.int64), P, block_sizes=Bs,
                                       block_tables=tables, slot_mappings=slots, **bufs)
        for B, row, sm in zip(Bs, tables, out["slot_mappings"]):
            # walk: tokens 0..P fill pages row[0], row[1], ... B at a time
            page_idx, off = 0, 0
            for _ in range(P):
                off += 1
                if off == B:
                    page_idx, off = page_idx + 1, 0
            assert sm[0] == int(row[page_idx]) * B + off


def test_input_prep_mrope_offset_and_is_token_ids():
    tables, bufs, slots = _prep_case(100, [16], mrope=True)
    itk = np.zeros(64, np.uint8)
    out = oracle.decode_input_prep(np.array([9], np.int64), 100, block_sizes=[16], block_tables=tables,
                                   slot_mappings=slots, mrope=True, mrope_delta=-37, is_token_ids=itk, **bufs)
    assert out["positions"][:, 0].tolist() == [63, 63, 63]
    assert out["is_token_ids"][0] == 1 and not out["is_token_ids"][1:].any()


# ---- several sequences in one prefill call -----------------------------------

def test_prefill_varlen_reduces_to_chunks_and_is_order_free():
    """One sequence reproduces prefill_chunk bitwise; reordering the sequences
    (rows and tables together) reorders the output rows and nothing else."""
    import workloads as W
    c = W.make_varlen_prefill_case("vl_pin", 7, [(5, 3), (0, 4), (17, 2)], 8, 12, hkv=1, hq=6, d=8,
                                   fill_bits=0)
    k, v = c.k_cache, c.v_cache
    for s, ch in enumerate(c.chunks):
        pos = np.arange(ch.start_pos, ch.start_pos + ch.q_len)
        k, v = oracle.kv_write(k, v, ch.k_new, ch.v_new, oracle.slot_mapping(pos, None, c.block_tables[s], 8))
    q = np.concatenate([ch.q for ch in c.chunks])
    lens = [ch.q_len for ch in c.chunks]
    cu = np.concatenate([[0], np.cumsum(lens)])
    used = [ch.start_pos + ch.q_len for ch in c.chunks]
    got = oracle.prefill_varlen(q, cu, used, True, k, v, c.block_tables, 8, 0.3)
    for s, ch in enumerate(c.chunks):
        want = oracle.prefill_chunk(ch.q, ch.start_pos, True, k, v, c.block_tables[s], 8, 0.3)
        assert np.array_equal(got[cu[s]:cu[s + 1]], want)
    order = [2, 0, 1]
    q2 = np.concatenate([c.chunks[i].q for i in order])
    cu2 = np.concatenate([[0], np.cumsum([lens[i] for i in order])])
    got2 = oracle.prefill_varlen(q2, cu2, [used[i] for i in order], True, k, v, c.block_tables[order], 8, 0.3)
    for j, i in enumerate(order):
        assert np.array_equal(got2[cu2[j]:cu2[j + 1]], got[cu[i]:cu[i + 1]])
