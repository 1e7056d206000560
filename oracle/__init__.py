"""fp64 CPU oracle for paged-KV grouped-query attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares
no code with the HIP library (``prefill_block_table_amd``) and imports
nothing from it; both sides take their inputs from ``workloads``.

What it computes is the plain definition: the pages state that paging,
page-contiguous decode and the vendor prefill all compute the same complete
causal attention, with no key skipped and the causal range not shortened
(page-alignment post, luanjiahao.me, §5 "From Page Table to Coalesced Load",
§7, §9 "Numerical Correctness").  So the oracle gathers logical K/V through
the block table and runs softmax(scale * q K^T) V in float64, one query head
at a time.

``gemv`` holds the decode-time bf16 M=1 linear layer y = W x, in float64
and in the library's fixed fp32 summation order (pinned by
``tests/test_oracle_gemv.py``).

Pinned by ``tests/test_oracle_pins.py`` (brute force, closed forms,
invariants, a library routine and the pages' printed page facts).
"""
from .paged_attention import (  # noqa: F401
    bf16_bits_to_f64,
    f64_to_bf16_bits,
    slot_mapping,
    kv_write,
    gather_kv,
    attend,
    decode,
    prefill_chunk,
    prefill_varlen,
)
from .input_prep import decode_input_prep  # noqa: F401
from .page_geometry import (  # noqa: F401
    attn_page_bytes_per_token,
    groups_in_page,
    page_bytes,
    required_page_tokens,
    smallest_aligned_page,
)
from .gemv import fp32_sum_error_bound, gemv_f64, gemv_fp32  # noqa: F401
