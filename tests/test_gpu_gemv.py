"""GPU parity: decode-time bf16 M=1 linear layer (pa_gemv_bf16) against the
oracle's fixed fp32 order, bit for bit, in both output types: small ragged
shapes (one row, a K that leaves lanes without a chunk, K above one register
pass, a row stride above K, K = 0), the three weight shapes of the
measurement post at full size, and repeat launches.  Every case is also
checked directly against the float64 definition: the fp32 output lies
within the standard fp32 summation error bound of the exact sum, and the
bf16 output within that bound plus half a bf16 unit in the last place."""
import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_util import bits, log, to_dev

pytestmark = pytest.mark.gpu


def _pa():
    import prefill_block_table_amd as pa
    return pa


def _check(W_bits, x_bits, ldw=None, seed_name=""):
    import torch
    pa = _pa()
    N, K = W_bits.shape
    log(f"gemv {seed_name} N={N} K={K} ldw={ldw}")
    if ldw is not None and ldw != K:
        pad = np.zeros((N, ldw), np.uint16)
        pad[:, :K] = W_bits
        pad[:, K:] = 0x7FC0                      # NaN beyond K: must never be read
        Wd = to_dev(pad)[:, :K]
    else:
        Wd = to_dev(W_bits)
    xd = to_dev(x_bits)
    yb = pa.gemv(Wd, xd)
    yf = pa.gemv(Wd, xd, out_dtype=torch.float32)
    torch.cuda.synchronize()
    want_f = oracle.gemv_fp32(W_bits, x_bits, "f32")
    want_b = oracle.gemv_fp32(W_bits, x_bits, "bf16")
    got_f = yf.cpu().numpy()
    got_b = bits(yb)
    nf = int(np.sum(got_f.view(np.uint32) != want_f.view(np.uint32)))
    nb = int(np.sum(got_b != want_b))
    log(f"  mismatches: f32 {nf}, bf16 {nb}")
    assert nf == 0 and nb == 0
    _check_against_definition(W_bits, x_bits, got_f, got_b)
    return Wd, xd, yb


def _check_against_definition(W_bits, x_bits, got_f, got_b):
    """|y - y_exact| within the fp32 error bound of this summation order (fp32
    output), plus half a bf16 ulp of the result (bf16 output), per row."""
    exact = oracle.gemv_f64(W_bits, x_bits)
    bound = oracle.fp32_sum_error_bound(W_bits, x_bits)
    err_f = np.abs(got_f.astype(np.float64) - exact)
    assert np.all(err_f <= bound), f"fp32 output outside the error bound: worst excess {float(np.max(err_f - bound))}"
    yb = oracle.bf16_bits_to_f64(got_b)
    # half a bf16 ulp of |y|: 2^(floor(log2|y|) - 8); subnormal quantum 2^-133
    mag = np.maximum(np.abs(yb), 2.0 ** -126)
    half_ulp = 2.0 ** (np.floor(np.log2(mag)) - 8)
    err_b = np.abs(yb - exact)
    assert np.all(err_b <= bound + half_ulp * (1 + 2.0 ** -8)), "bf16 output outside bound + half ulp"
    rel = float(np.max(err_f / np.maximum(bound, 1e-300))) if bound.size else 0.0
    log(f"  vs float64 definition: max |err| fp32 {float(err_f.max()) if err_f.size else 0:.3e}, "
        f"largest fraction of the bound {rel:.3f}")


SMALL = [(1, 8), (7, 520), (9, 5120), (13, 1032), (5, 8192), (3, 16392), (64, 64), (33, 4096)]


@pytest.mark.parametrize("N,K", SMALL)
def test_gemv_small_bit_exact(N, K):
    W, x = wl.make_gemv_case(100 + N, N, K, w_std=1.0)
    _check(W, x, seed_name="small")


def test_gemv_row_stride_above_k():
    W, x = wl.make_gemv_case(7, 21, 1032)
    _check(W, x, ldw=1040, seed_name="strided")


def test_gemv_k_zero_gives_positive_zero():
    import torch
    pa = _pa()
    log("gemv K=0")
    W = torch.empty((5, 0), dtype=torch.bfloat16, device="cuda:0")
    x = torch.empty((0,), dtype=torch.bfloat16, device="cuda:0")
    y = pa.gemv(W, x, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert np.all(y.cpu().numpy().view(np.uint32) == 0)


@pytest.mark.parametrize("N,K", wl.GEMV_SHAPES)
def test_gemv_full_shapes_bit_exact_and_repeatable(N, K):
    import torch
    pa = _pa()
    W, x = wl.make_gemv_case(N, N, K)
    Wd, xd, y0 = _check(W, x, seed_name="full")
    for _ in range(3):
        y1 = pa.gemv(Wd, xd)
        torch.cuda.synchronize()
        assert torch.equal(y1.view(torch.int16), y0.view(torch.int16))
