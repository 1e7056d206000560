"""Single-token decode input preparation, the plain definition (test
infrastructure only).

Single-token input-prep post (jsqmd.com/news/1214744), §2: with one request
that advances by one token, input_ids[0] is the previous step's sampled
token, the position is the number of tokens already computed,
query_start_loc is [0, 1, 1, ...], seq_lens is [position + 1, 0, 0, ...],
the discard mask is all false; §3.2: each KV-cache group's slot is
block_table[position // B] * B + position % B; §5: with M-RoPE the position
is written to all three rows, with prompt embeddings is_token_ids[0] is set.
The M-RoPE offset (vLLM's per-request M-RoPE position delta, 0 for a text-only
request) is this build's reading; the post writes the three rows without
naming it.

Written from the generic definitions rather than the closed forms: the
scheduled-token counts of the max_num_reqs request slots are [1, 0, 0, ...];
query_start_loc is their exclusive-then-inclusive prefix sum and seq_lens is
computed tokens + scheduled tokens per request.
"""
from __future__ import annotations

import numpy as np

from .paged_attention import slot_mapping


def decode_input_prep(sampled_token_ids, position: int, input_ids, positions, query_start_loc,
                      seq_lens, discard_request_mask, block_sizes=(), block_tables=(),
                      slot_mappings=(), mrope: bool = False, mrope_delta: int = 0,
                      is_token_ids=None):
    """Returns new copies of every output buffer (the given arrays are the
    buffers' contents before the step; entries the step does not define are
    returned unchanged).  block_tables[g] is group g's block-table row."""
    out = {}
    ids = np.array(input_ids, copy=True)
    ids[0] = int(sampled_token_ids[0])
    out["input_ids"] = ids
    pos = np.array(positions, copy=True)
    if mrope:
        pos[:, 0] = position + mrope_delta
    else:
        pos[0] = position
    out["positions"] = pos
    n_slots = len(seq_lens)
    scheduled = np.zeros(max(n_slots, len(query_start_loc) - 1), dtype=np.int64)
    scheduled[0] = 1                                  # one request, one token
    computed = np.zeros_like(scheduled)
    computed[0] = position
    qsl = np.concatenate([[0], np.cumsum(scheduled)])[:len(query_start_loc)]
    out["query_start_loc"] = qsl.astype(np.asarray(query_start_loc).dtype)
    out["seq_lens"] = (computed + scheduled)[:n_slots].astype(np.asarray(seq_lens).dtype)
    out["discard_request_mask"] = np.zeros_like(np.asarray(discard_request_mask))
    if is_token_ids is not None:
        itk = np.array(is_token_ids, copy=True)
        itk[0] = 1
        out["is_token_ids"] = itk
    sms = []
    for B, row, sm in zip(block_sizes, block_tables, slot_mappings):
        new = np.array(sm, copy=True)
        new[0] = slot_mapping(np.array([position], dtype=np.int64), None,
                              np.asarray(row, dtype=np.int64)[None, :], int(B))[0]
        sms.append(new)
    out["slot_mappings"] = sms
    return out
