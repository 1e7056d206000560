"""Page-size derivation of the C ABI (pa_page_size_for_hybrid, host-only
arithmetic, no device) against the oracle's rendering of the page-alignment
post's section 3 formula: exact integer equality."""
import ctypes

import numpy as np
import pytest

import oracle

pa = pytest.importorskip("prefill_block_table_amd")


def _codes():
    import os
    import re
    hdr = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "pa.h")
    return {m[0]: int(m[1]) for m in re.findall(r"#define (PA_[A-Z_]+) (-?\d+)", open(hdr).read())}


def test_printed_pages():
    per_tok = oracle.attn_page_bytes_per_token(4, 256, 2)
    for m in (3_145_729, 3_180_000, 3_211_264):
        assert pa.page_size_for_hybrid(m, per_tok, 16) == 784
        assert pa.page_size_for_hybrid(m, per_tok, 64) == 832


def test_matches_oracle_on_a_sweep():
    rng = np.random.Generator(np.random.PCG64(5))
    cases = [(int(rng.integers(1, 1 << 40)), int(rng.integers(1, 1 << 16)), int(a))
             for a in rng.choice([1, 2, 16, 64, 128, 256], size=2000)]
    cases += [(m, 4096, a) for a in (16, 64) for m in range(3_145_000, 3_215_000, 977)]
    cases += [(1, 1, 1), (4096 * 64, 4096, 64), (4096 * 64 + 1, 4096, 64)]
    for m, per_tok, align in cases:
        want = oracle.required_page_tokens(m, per_tok, align)
        if want > 2**31 - 1:
            with pytest.raises(pa.PAError):
                pa.page_size_for_hybrid(m, per_tok, align)
        else:
            assert pa.page_size_for_hybrid(m, per_tok, align) == want, (m, per_tok, align)


def test_errors():
    C = _codes()
    out = ctypes.c_int32(0)
    L = pa.lib
    assert L.pa_page_size_for_hybrid(3_200_000, 4096, 64, None) == C["PA_ERR_NULL"]
    for args in ((0, 4096, 64), (3_200_000, 0, 64), (3_200_000, 4096, 0), (-1, 4096, 64)):
        assert L.pa_page_size_for_hybrid(*args, ctypes.byref(out)) == C["PA_ERR_SIZE"]
    # a result beyond int32 and an overflowing group size are rejected
    assert L.pa_page_size_for_hybrid(1 << 62, 1, 64, ctypes.byref(out)) == C["PA_ERR_SIZE"]
    assert L.pa_page_size_for_hybrid(1 << 40, 1 << 62, 64, ctypes.byref(out)) == C["PA_ERR_SIZE"]
