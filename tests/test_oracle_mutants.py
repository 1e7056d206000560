"""Plant plausible mistakes in the oracle and check that the pins catch them.

Each mutant replaces one oracle function (on the CPU, through monkeypatch)
with a version that carries one typical slip: a dropped scale, a wrong
query-to-KV-head map, an off-by-one causal bound, swapped K and V, a block
table that is not consulted, a wrong page offset, a decode that drops the
newest key, a slot formula with page and offset swapped, a KV write one row
off.  The pins of ``test_oracle_pins.py`` must fail for every one.  Further
slips are planted in the single-token input prep (seq_lens without the +1, a
running query_start_loc, the next page's slot, M-RoPE on one row only, the
position as the token id) and in the page-size derivation (floor for ceiling,
no rounding to the alignment, one group too many on an exact fit, only K's
bytes per token).
"""
import numpy as np
import pytest

import oracle
from oracle import paged_attention as pa
import test_oracle_pins as pins

_orig_attend = pa.attend
_orig_gather = pa.gather_kv
_orig_decode = pa.decode


def m_drop_scale(q, qpos, K, V, scale, causal=True, return_weights=False):
    return _orig_attend(q, qpos, K, V, 1.0, causal, return_weights)


def m_head_modulo(q, qpos, K, V, scale, causal=True, return_weights=False):
    Hq, Hkv = np.shape(q)[1], np.shape(K)[1]
    idx = [h % Hkv for h in range(Hq)]
    return _orig_attend(q, qpos, np.asarray(K)[:, idx], np.asarray(V)[:, idx], scale, causal,
                        return_weights)


def m_causal_strict(q, qpos, K, V, scale, causal=True, return_weights=False):
    return _orig_attend(q, np.asarray(qpos) - 1, K, V, scale, causal, return_weights)


def m_swap_kv(q, qpos, K, V, scale, causal=True, return_weights=False):
    return _orig_attend(q, qpos, V, K, scale, causal, return_weights)


def m_no_table(cache, block_table_row, seq_len, block_size):
    return _orig_gather(cache, np.arange(len(block_table_row)), seq_len, block_size)


def m_offset_shift(cache, block_table_row, seq_len, block_size):
    t = np.arange(seq_len)
    return np.asarray(cache)[np.asarray(block_table_row)[t // block_size],
                             (t + 1) % block_size]


def m_decode_drops_newest(q, k_cache, v_cache, block_tables, seq_lens, block_size, scale,
                          seqs=None):
    lens = np.maximum(np.asarray(seq_lens) - 1, 1)
    return _orig_decode(q, k_cache, v_cache, block_tables, lens, block_size, scale, seqs)


def m_slot_swapped(positions, token_seq, block_tables, block_size):
    pos = np.asarray(positions, np.int64)
    seq = np.zeros_like(pos) if token_seq is None else np.asarray(token_seq, np.int64)
    bt = np.asarray(block_tables)
    bt = bt[None] if bt.ndim == 1 else bt
    return bt[seq, pos % bt.shape[1]].astype(np.int64) * block_size + pos // block_size


def m_kv_write_off_by_one(k_cache, v_cache, k_new, v_new, slots):
    return pa.__dict__["_real_kv_write"](k_cache, v_cache, k_new, v_new,
                                        np.asarray(slots, np.int64) + 1)


PIN_CALLS = [
    lambda: pins.test_decode_vs_brute_force(5, (12, 2, 8)),
    lambda: pins.test_decode_vs_brute_force(3, (6, 1, 4)),
    lambda: pins.test_prefill_vs_brute_force(5, 7, 6, True),
    lambda: pins.test_prefill_vs_brute_force(4, 0, 9, False),
    lambda: pins.test_full_shape_vs_brute_force_tiny_context(),
    lambda: pins.test_zero_query_gives_prefix_mean(),
    lambda: pins.test_one_token_context_returns_v_exactly(),
    lambda: pins.test_gqa_equals_mha_with_repeated_kv(),
    lambda: pins.test_slot_mapping_brute_force(16),
    lambda: pins.test_decode_metadata_golden(),
    lambda: pins.test_kv_write_bytes(),
]

MUTANTS = {
    "drop_scale": ("attend", m_drop_scale),
    "head_modulo": ("attend", m_head_modulo),
    "causal_strict": ("attend", m_causal_strict),
    "swap_kv": ("attend", m_swap_kv),
    "no_table": ("gather_kv", m_no_table),
    "offset_shift": ("gather_kv", m_offset_shift),
    "decode_drops_newest": ("decode", m_decode_drops_newest),
    "slot_swapped": ("slot_mapping", m_slot_swapped),
    "kv_write_off_by_one": ("kv_write", m_kv_write_off_by_one),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, monkeypatch):
    fn_name, mutant = MUTANTS[name]
    monkeypatch.setitem(pa.__dict__, "_real_kv_write", pa.kv_write)
    monkeypatch.setattr(pa, fn_name, mutant)
    monkeypatch.setattr(oracle, fn_name, mutant)
    caught = 0
    for call in PIN_CALLS:
        try:
            call()
        except (AssertionError, ValueError, IndexError):
            caught += 1
    assert caught >= 1, f"mutant {name} passed every pin"


# ---- input preparation -------------------------------------------------------

_orig_prep = oracle.decode_input_prep


def _prep_mutant(edit):
    def f(*args, **kw):
        out = _orig_prep(*args, **kw)
        edit(out, args, kw)
        return out
    return f


def _seq_lens_no_plus_one(out, args, kw):
    out["seq_lens"][0] -= 1


def _qsl_running_index(out, args, kw):
    out["query_start_loc"][:] = np.arange(len(out["query_start_loc"]))


def _slot_next_page(out, args, kw):
    pos = args[1]
    for B, row, sm in zip(kw["block_sizes"], kw["block_tables"], out["slot_mappings"]):
        sm[0] = int(row[pos // B + 1]) * B + pos % B


def _mrope_first_row_only(out, args, kw):
    if kw.get("mrope"):
        out["positions"][1:, 0] = -7


def _input_id_from_position(out, args, kw):
    out["input_ids"][0] = args[1]


PREP_MUTANTS = {
    "seq_lens_no_plus_one": _seq_lens_no_plus_one,
    "qsl_running_index": _qsl_running_index,
    "slot_next_page": _slot_next_page,
    "mrope_first_row_only": _mrope_first_row_only,
    "input_id_from_position": _input_id_from_position,
}
PREP_PINS = [pins.test_input_prep_printed_closed_forms, pins.test_input_prep_slot_matches_gather,
             pins.test_input_prep_mrope_offset_and_is_token_ids]


@pytest.mark.parametrize("name", sorted(PREP_MUTANTS))
def test_input_prep_pins_catch_mutant(name, monkeypatch):
    monkeypatch.setattr(oracle, "decode_input_prep", _prep_mutant(PREP_MUTANTS[name]))
    caught = 0
    for call in PREP_PINS:
        try:
            call()
        except (AssertionError, ValueError, IndexError):
            caught += 1
    assert caught >= 1, f"mutant {name} passed every pin"


# ---- page-size derivation ----------------------------------------------------

def _page_floor(m, per_tok, align):
    return (m // (align * per_tok)) * align


def _page_no_alignment(m, per_tok, align):
    return -(-m // per_tok)


def _page_always_one_more(m, per_tok, align):
    return (m // (align * per_tok) + 1) * align


def _page_k_bytes_only(m, per_tok, align):
    return -(-m // (align * (per_tok // 2))) * align


PAGE_MUTANTS = {
    "floor_not_ceil": _page_floor,
    "no_alignment": _page_no_alignment,
    "always_one_more_group": _page_always_one_more,
    "k_bytes_only": _page_k_bytes_only,
}
PAGE_PINS = [pins.test_page_derivation_reproduces_printed_pages, pins.test_page_derivation_brute_force]


@pytest.mark.parametrize("name", sorted(PAGE_MUTANTS))
def test_page_pins_catch_mutant(name, monkeypatch):
    monkeypatch.setattr(oracle, "required_page_tokens", PAGE_MUTANTS[name])
    caught = 0
    for call in PAGE_PINS:
        try:
            call()
        except (AssertionError, ValueError, IndexError, ZeroDivisionError):
            caught += 1
    assert caught >= 1, f"mutant {name} passed every pin"


def test_page_mutant_harness_passes_unmutated():
    for call in PAGE_PINS:
        call()
