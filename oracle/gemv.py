"""bf16 M=1 linear layer y = W x, two plain definitions (test infrastructure only).

Long-context inference measurement post (luanjiahao.me, 2026-07-17), §4: a
decode-time linear layer with one input row computes y[j] = sum_k x[k] W[j, k]
from bf16 weights and a bf16 input with fp32 accumulation; §5: weight shapes
14336, 16384 and 34816 x 5120, and two row blockings of one kernel give
bitwise identical outputs.

``gemv_f64`` is the definition in float64.  Every bf16 x bf16 product is exact
in float64 (16 significant bits); the sum rounds, with a relative error far
below fp32's, so it serves as the exact value within fp32 error bounds.

``gemv_fp32`` fixes one fp32 summation order, the reading of "fp32
accumulation" that this library uses, so that results can be compared bit
for bit.  The order, in the terms of the definition:
  * a row of K elements is cut into 16-byte chunks of 8 consecutive elements
    (chunk c holds k = 8c .. 8c + 7);
  * 64 partial sums ("lanes") start at +0.0; lane l takes chunks l, l + 64,
    l + 128, ... in increasing order and, inside a chunk, the elements in
    increasing k (a bf16 pair: the even k, then the odd k), adding each exact
    product x[k] * W[j, k] to its fp32 sum with one rounding;
  * the 64 lane sums are combined by a butterfly: for d = 32, 16, 8, 4, 2, 1,
    every lane l replaces its sum by fp32(sum_l + sum_(l xor d)); after the six
    steps every lane holds the same value, which is y[j] in fp32;
  * the bf16 output is that value rounded to nearest, ties to even.
Adding an exact product with one rounding is what a fused multiply-add does;
it equals fp32(product) + acc in fp32 whenever the product is exactly an fp32
number, which ``gemv_fp32`` checks (it is, unless a product falls below fp32's
normal range).
"""
from __future__ import annotations

import numpy as np

from .paged_attention import bf16_bits_to_f64, f64_to_bf16_bits

LANES = 64
CHUNK = 8
BUTTERFLY = (32, 16, 8, 4, 2, 1)


def _bf16_to_f32(bits) -> np.ndarray:
    """bf16 bit patterns to float32: the bits are the top half of an fp32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def gemv_f64(W_bits, x_bits) -> np.ndarray:
    """y[j] = sum_k x[k] W[j, k] in float64 from bf16 bit patterns [N, K], [K]."""
    W = bf16_bits_to_f64(W_bits)
    x = bf16_bits_to_f64(x_bits)
    if W.ndim != 2 or x.shape != (W.shape[1],):
        raise ValueError("W must be [N, K] and x [K]")
    return W @ x


def gemv_fp32(W_bits, x_bits, out: str = "bf16") -> np.ndarray:
    """y = W x in the fixed fp32 order above; ``out`` is "f32" or "bf16"
    (then the result is uint16 bf16 bit patterns)."""
    W_bits = np.asarray(W_bits, dtype=np.uint16)
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    if W_bits.ndim != 2 or x_bits.shape != (W_bits.shape[1],):
        raise ValueError("W must be [N, K] and x [K]")
    N, K = W_bits.shape
    if K % CHUNK:
        raise ValueError("K must be a multiple of 8")
    W32 = _bf16_to_f32(W_bits)
    x32 = _bf16_to_f32(x_bits)
    prod = W32 * x32[None, :]                       # fp32 products
    # A product of two bf16 values has at most 16 significant bits, so it is
    # an fp32 number unless it lands below fp32's normal range.
    tiny = (np.abs(prod) < np.float32(2.0 ** -126)) & (W32 != 0) & (x32 != 0)[None, :]
    if tiny.any():
        raise ValueError("a bf16 product is not exact in fp32 (fp32 underflow)")

    nchunks = K // CHUNK
    chunks = prod.reshape(N, nchunks, CHUNK)        # chunk c = elements 8c .. 8c + 7
    acc = np.zeros((N, LANES), dtype=np.float32)
    lane = np.arange(LANES)
    for first in range(0, nchunks, LANES):          # lane l takes chunk first + l
        live = min(LANES, nchunks - first)
        block = chunks[:, first:first + live, :]
        for e in range(CHUNK):                      # elements of the chunk in order
            acc[:, :live] = acc[:, :live] + block[:, :, e]
    for d in BUTTERFLY:
        acc = acc + acc[:, lane ^ d]
    y32 = acc[:, 0].copy()
    if out == "f32":
        return y32
    if out == "bf16":
        return f64_to_bf16_bits(y32.astype(np.float64))
    raise ValueError("out must be 'f32' or 'bf16'")


def fp32_sum_error_bound(W_bits, x_bits) -> np.ndarray:
    """Per row, the standard bound on |fp32 result - exact| for this order:
    every term passes through at most 8 * ceil(K / 512) + 6 roundings, each of
    relative size at most u = 2^-24, so |error| <= gamma_n * sum_k |x_k W_jk|
    with n that count and gamma_n = n u / (1 - n u)."""
    W = np.abs(bf16_bits_to_f64(W_bits))
    x = np.abs(bf16_bits_to_f64(x_bits))
    K = W.shape[1]
    n = CHUNK * (-(-(K // CHUNK) // LANES)) + len(BUTTERFLY)
    u = 2.0 ** -24
    return (n * u / (1.0 - n * u)) * (W @ x)
