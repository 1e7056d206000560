"""GPU parity sweep over seeded random shapes, weighted toward the page sizes
where the kernels change behaviour: pages below, at and just above the
64-token key group (prefill groups then span pages or stay inside one page),
around the 16-token decode step, the measured 784 / 832 / 1024 and their
neighbours, and page 1.  Prefill chunks (one or two, causal or not, 1-8 KV
heads), several-sequence prefill batches (1-12 sequences, empty ones among
them) and decode batches (1-8 sequences, with or without the appended token)
are each compared with the oracle on every output row."""
import numpy as np
import pytest

import workloads as W
from gpu_util import compare, log

pytestmark = pytest.mark.gpu

PAGES = [1, 2, 7, 15, 16, 31, 32, 33, 48, 63, 64, 65, 66, 96, 100, 127, 128, 129, 130, 191, 192,
         200, 255, 256, 257, 500, 783, 784, 785, 832, 1000, 1023, 1024, 1025]
N_PREFILL, N_VARLEN, N_DECODE = 96, 48, 96


def _page(rng):
    return int(rng.choice(PAGES)) if rng.random() < 0.8 else int(rng.integers(1, 1400))


@pytest.mark.parametrize("i", range(N_PREFILL))
def test_prefill_chunks(i):
    import test_gpu_prefill as TP
    rng = np.random.default_rng(31_000 + i)
    B = _page(rng)
    hkv = int(rng.choice([1, 2, 3, 4, 4, 4, 8]))
    start = int(rng.integers(0, 3001)) if rng.random() < 0.8 else int(rng.integers(0, 64))
    chunks = [(start, int(rng.integers(1, 501)))]
    if rng.random() < 0.4:
        chunks.append((start + chunks[0][1], int(rng.integers(1, 301))))
    causal = bool(rng.random() < 0.85)
    end = chunks[-1][0] + chunks[-1][1]
    c = W.make_prefill_case(f"sweep_pf{i}_b{B}_hkv{hkv}", 32_000 + i, chunks, B, -(-end // B) + 2,
                            causal=causal, hkv=hkv, hq=6 * hkv)
    log(f"{c.name} chunks={chunks} causal={causal}")
    for j, (g, r) in enumerate(zip(TP.run_chunks_gpu(c), TP.run_chunks_oracle(c))):
        compare(g, r, f"{c.name}[{j}]")


@pytest.mark.parametrize("i", range(N_VARLEN))
def test_prefill_varlen_batches(i):
    import test_gpu_prefill as TP
    rng = np.random.default_rng(33_000 + i)
    B = _page(rng)
    hkv = int(rng.choice([1, 2, 4, 4]))
    seqs = [(int(rng.integers(0, 2001)), int(rng.integers(0, 301))) for _ in range(int(rng.integers(1, 13)))]
    seqs = [(max(s0, 1) if n == 0 else s0, n) for s0, n in seqs]   # every sequence holds a token
    if all(n == 0 for _, n in seqs):
        seqs[0] = (seqs[0][0], 1)
    causal = bool(rng.random() < 0.85)
    pages = sum(-(-(s0 + n) // B) for s0, n in seqs)
    c = W.make_varlen_prefill_case(f"sweep_vl{i}_b{B}_hkv{hkv}", 34_000 + i, seqs, B, pages + 4,
                                   causal=causal, hkv=hkv, hq=6 * hkv)
    log(f"{c.name} seqs={seqs} causal={causal}")
    TP._check_varlen(c, causal)


@pytest.mark.parametrize("i", range(N_DECODE))
def test_decode_batches(i):
    import test_gpu_decode as TD
    rng = np.random.default_rng(35_000 + i)
    B = _page(rng)
    hkv = int(rng.choice([1, 2, 3, 4, 4, 5, 6, 8]))
    lens = [int(x) for x in rng.integers(1, 5001, size=int(rng.integers(1, 9)))]
    append = bool(rng.integers(0, 2))
    pages = sum(-(-(n + 1) // B) for n in lens) + 2
    c = W.make_decode_case(f"sweep_dec{i}_b{B}_hkv{hkv}", 36_000 + i, lens, B, pages,
                           write_new_token=append, hkv=hkv, hq=6 * hkv)
    log(f"{c.name} lens={lens} append={append}")
    if append:
        TD._check_append(c)
    else:
        compare(TD.run_gpu(c), TD.run_oracle(c), c.name)
