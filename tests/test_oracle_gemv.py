"""Pins for the oracle's decode-time linear layer y = W x (``oracle/gemv.py``).

The definition (long-context inference measurement post, luanjiahao.me
2026-07-17, §4): y[j] = sum_k x[k] W[j, k], bf16 weights and input, fp32
accumulation.  ``gemv_fp32`` fixes one fp32 order; these tests tie it to
things other than itself:
  * the exact sum (math.fsum of exact products) within the standard
    floating-point error bound of that order, on ragged K;
  * integer inputs, where every partial sum is exact, against an integer
    matrix product;
  * the bf16 output against torch's float32 -> bfloat16 rounding;
  * two hand-derived values whose result depends on the order (derivations
    in the tests), one for the order inside a lane, one for the butterfly;
  * invariances: row permutation, scaling by a power of two.
Then plausible slips are planted in a copy of the order (reversed elements,
reversed chunks, contiguous chunk ranges per lane, reversed or sequential
lane combination, a dropped ragged chunk, x shifted by one, truncating bf16
rounding, the transposed weight) and each must fail one of the pins.
"""
import math

import numpy as np
import pytest
import torch

import oracle

BIG = 2.0 ** 24


def _bits(values) -> np.ndarray:
    """bf16 bit patterns of values that bf16 holds exactly."""
    f = np.asarray(values, dtype=np.float32)
    u = f.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not exact in bf16"
    return (u >> 16).astype(np.uint16)


def _rand(seed, N, K, w_std=0.02):
    rng = np.random.Generator(np.random.PCG64(seed))
    W = rng.standard_normal((N, K)).astype(np.float32) * np.float32(w_std)
    x = rng.standard_normal(K).astype(np.float32)
    # truncate to bf16 (any bf16 input will do for these pins)
    return ((W.view(np.uint32) >> 16).astype(np.uint16), (x.view(np.uint32) >> 16).astype(np.uint16))


def _f(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _exact(W_bits, x_bits):
    W, x = _f(W_bits), _f(x_bits)
    return np.array([math.fsum(W[j] * x) for j in range(W.shape[0])])


# ---------------------------------------------------------------- pins

@pytest.mark.parametrize("K", [8, 504, 512, 520, 1032, 5120])
def test_gemv_within_error_bound_of_exact_sum(K):
    W, x = _rand(K, 9, K)
    exact = _exact(W, x)
    y32 = oracle.gemv_fp32(W, x, "f32").astype(np.float64)
    bound = oracle.fp32_sum_error_bound(W, x)
    assert np.all(np.abs(y32 - exact) <= bound)
    # the float64 definition agrees with the exact sum to float64 rounding
    assert np.allclose(oracle.gemv_f64(W, x), exact, rtol=1e-13, atol=1e-300)


def test_gemv_square_not_transposed():
    W, x = _rand(7, 64, 64, w_std=1.0)
    exact = _exact(W, x)
    y32 = oracle.gemv_fp32(W, x, "f32").astype(np.float64)
    assert np.all(np.abs(y32 - exact) <= oracle.fp32_sum_error_bound(W, x))


def test_gemv_integer_inputs_are_exact():
    rng = np.random.Generator(np.random.PCG64(11))
    N, K = 33, 5120
    Wi = rng.integers(-8, 9, size=(N, K))
    xi = rng.integers(-8, 9, size=K)
    want = Wi @ xi            # |partial sums| <= 64 * 5120 < 2^24: every fp32 step exact
    y32 = oracle.gemv_fp32(_bits(Wi), _bits(xi), "f32")
    assert np.array_equal(y32.astype(np.int64), want)


def test_gemv_bf16_output_is_torch_rounding():
    W, x = _rand(5, 300, 1032, w_std=1.0)
    y32 = oracle.gemv_fp32(W, x, "f32")
    yb = oracle.gemv_fp32(W, x, "bf16")
    ref = torch.from_numpy(y32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(yb, ref)


def test_gemv_order_inside_a_lane_hand_value():
    # K = 1024: 128 chunks, lane 0 owns chunks 0 and 64.  x = 1.  Row 0 holds
    # 2^24 at k = 0 and 1.0 at k = 1..7 (rest of chunk 0) and k = 512..519
    # (chunk 64).  Lane 0 starts with 2^24; each following +1 lands halfway
    # between 2^24 and 2^24 + 2 and rounds to the even 2^24, so lane 0 ends at
    # exactly 2^24 and so does y (other lanes are 0).  The exact sum is
    # 2^24 + 15.  Reversed elements, reversed chunks, or lane 0 owning chunks
    # 0 and 1 instead each give 2^24 + 8.
    K = 1024
    w = np.zeros(K)
    w[0] = BIG
    w[1:8] = 1.0
    w[512:520] = 1.0
    W = _bits(np.stack([w, np.ones(K)]))
    x = _bits(np.ones(K))
    y32 = oracle.gemv_fp32(W, x, "f32")
    assert y32[0] == np.float32(BIG)
    assert y32[1] == np.float32(K)


def test_gemv_butterfly_order_hand_value():
    # K = 512: one chunk per lane; lane l's sum is W[0, 8l] (x = 1).  Lane
    # sums: v0 = 2^24, v2 = v33 = v34 = 1, the rest 0.  Distance 32 first:
    # lane 0 = 2^24, lane 1 = v1 + v33 = 1, lane 2 = v2 + v34 = 2; distances
    # 16, 8, 4 add zeros to lanes 0..3; distance 2: lane 0 = 2^24 + 2 (exact),
    # lane 1 = 1; distance 1: 2^24 + 3 is a tie between 2^24 + 2 and 2^24 + 4
    # and goes to the even 2^24 + 4.  Distance 1 first would give 2^24 + 2, a
    # sequential sum over lanes 2^24, the exact sum 2^24 + 3.
    K = 512
    w = np.zeros(K)
    w[0] = BIG
    for lane in (2, 33, 34):
        w[8 * lane] = 1.0
    y32 = oracle.gemv_fp32(_bits(w[None]), _bits(np.ones(K)), "f32")
    assert y32[0] == np.float32(BIG + 4)


def test_gemv_row_permutation_and_power_of_two_scale():
    W, x = _rand(3, 50, 520, w_std=1.0)
    y = oracle.gemv_fp32(W, x, "f32")
    perm = np.random.Generator(np.random.PCG64(4)).permutation(50)
    assert np.array_equal(oracle.gemv_fp32(W[perm], x, "f32"), y[perm])
    x2 = _bits(_f(x) * 4.0)
    assert np.array_equal(oracle.gemv_fp32(W, x2, "f32"), y * np.float32(4.0))


def test_gemv_edge_cases():
    W = np.zeros((3, 0), np.uint16)
    x = np.zeros(0, np.uint16)
    y = oracle.gemv_fp32(W, x, "f32")
    assert y.shape == (3,) and np.all(y == 0) and not np.any(np.signbit(y))
    with pytest.raises(ValueError):
        oracle.gemv_fp32(np.zeros((2, 12), np.uint16), np.zeros(12, np.uint16))
    with pytest.raises(ValueError):   # 2^-70 * 2^-70 is below fp32's normal range
        oracle.gemv_fp32(_bits(np.full((1, 8), 2.0 ** -70)), _bits(np.full(8, 2.0 ** -70)))


PINS = [
    lambda: test_gemv_within_error_bound_of_exact_sum(520),
    lambda: test_gemv_within_error_bound_of_exact_sum(5120),
    test_gemv_square_not_transposed,
    test_gemv_integer_inputs_are_exact,
    test_gemv_bf16_output_is_torch_rounding,
    test_gemv_order_inside_a_lane_hand_value,
    test_gemv_butterfly_order_hand_value,
    test_gemv_row_permutation_and_power_of_two_scale,
]


# ------------------------------------------------------------- mutants

def _variant(W_bits, x_bits, out="bf16", *, elems=None, chunk_rev=False, contiguous=False,
             butterfly=(32, 16, 8, 4, 2, 1), sequential=False, drop_tail=False, x_shift=False,
             truncate=False, transpose=False):
    W = _f(W_bits).astype(np.float32)
    if transpose:
        W = W.T.copy()
    x = _f(x_bits).astype(np.float32)
    if x_shift:
        x = np.roll(x, 1)
    N, K = W.shape
    nch = K // 8
    rounds = -(-nch // 64)
    acc = np.zeros((N, 64), np.float32)
    for lane in range(64):
        if contiguous:
            own = [c for c in range(lane * rounds, (lane + 1) * rounds) if c < nch]
        else:
            own = [c for c in range(lane, nch, 64)]
        if drop_tail and nch % 64:
            own = [c for c in own if c < nch - nch % 64]
        if chunk_rev:
            own = own[::-1]
        for c in own:
            for e in (elems or range(8)):
                k = 8 * c + e
                acc[:, lane] = acc[:, lane] + W[:, k] * x[k]
    if sequential:
        y = np.zeros(N, np.float32)
        for lane in range(64):
            y = y + acc[:, lane]
    else:
        idx = np.arange(64)
        for d in butterfly:
            acc = acc + acc[:, idx ^ d]
        y = acc[:, 0]
    if out == "f32":
        return y
    u = y.view(np.uint32)
    if truncate:
        return (u >> 16).astype(np.uint16)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


MUTANTS = {
    "reversed_elements": dict(elems=range(7, -1, -1)),
    "reversed_chunks": dict(chunk_rev=True),
    "contiguous_lanes": dict(contiguous=True),
    "reversed_butterfly": dict(butterfly=(1, 2, 4, 8, 16, 32)),
    "sequential_lanes": dict(sequential=True),
    "dropped_tail_chunk": dict(drop_tail=True),
    "x_shifted": dict(x_shift=True),
    "truncating_bf16": dict(truncate=True),
    "transposed_W": dict(transpose=True),
}


def test_unmutated_variant_matches_oracle():
    W, x = _rand(9, 17, 1032, w_std=1.0)
    assert np.array_equal(_variant(W, x, "f32"), oracle.gemv_fp32(W, x, "f32"))
    assert np.array_equal(_variant(W, x), oracle.gemv_fp32(W, x))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_gemv_pins_catch_mutant(name, monkeypatch):
    kw = MUTANTS[name]
    monkeypatch.setattr(oracle, "gemv_fp32", lambda W, x, out="bf16": _variant(W, x, out, **kw))
    failed = 0
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            failed += 1
    assert failed > 0, f"mutant {name} passed every pin"
