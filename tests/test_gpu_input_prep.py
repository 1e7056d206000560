"""GPU parity: single-token decode input preparation (pa_decode_input_prep)
against the oracle, bit-exact on every output buffer, including the entries
the step must leave untouched (poison before, compared after)."""
import numpy as np
import pytest

import oracle
from gpu_util import log, to_dev

pytestmark = pytest.mark.gpu

POISON = -7


def _pa():
    import prefill_block_table_amd as pa
    return pa


def _run(position, block_sizes, n_tokens=64, n_reqs=16, mrope=False, delta=0, with_itk=False,
         seed=0, token=151_643):
    import torch
    pa = _pa()
    log(f"input prep: pos={position} B={block_sizes} mrope={mrope} delta={delta} itk={with_itk}")
    rng = np.random.Generator(np.random.PCG64(seed))
    tables = [rng.permutation(1 << 20)[: -(-(position + 1) // B) + 2].astype(np.int32)
              for B in block_sizes]
    host = dict(
        input_ids=np.full(n_tokens, POISON, np.int32),
        positions=np.full((3, n_tokens + 1) if mrope else n_tokens, POISON, np.int64),
        query_start_loc=np.full(n_reqs + 1, POISON, np.int32),
        seq_lens=np.full(n_reqs, POISON, np.int32),
        discard_request_mask=np.ones(n_reqs, np.uint8),
    )
    itk = np.zeros(n_tokens, np.uint8) if with_itk else None
    slots = [np.full(n_tokens, POISON, np.int64) for _ in block_sizes]
    sampled = np.array([token, 99], np.int64)

    dev = {k: to_dev(v) for k, v in host.items()}
    d_itk = to_dev(itk) if with_itk else None
    d_tables = [to_dev(t) for t in tables]
    d_slots = [to_dev(s) for s in slots]
    G = len(block_sizes)
    kw = {}
    if G:
        kw = dict(block_sizes=to_dev(np.array(block_sizes, np.int32)),
                  block_table_ptrs=torch.tensor([t.data_ptr() for t in d_tables], dtype=torch.int64,
                                                device="cuda"),
                  slot_mapping_ptrs=torch.tensor([s.data_ptr() for s in d_slots], dtype=torch.int64,
                                                 device="cuda"))
    pa.decode_input_prep(to_dev(sampled), position, dev["input_ids"], dev["positions"],
                         dev["query_start_loc"], dev["seq_lens"], dev["discard_request_mask"],
                         mrope=mrope, mrope_delta=delta, is_token_ids=d_itk, **kw)
    torch.cuda.synchronize()
    want = oracle.decode_input_prep(sampled, position, block_sizes=block_sizes, block_tables=tables,
                                    slot_mappings=slots, mrope=mrope, mrope_delta=delta,
                                    is_token_ids=itk, **host)
    for k in host:
        got = dev[k].cpu().numpy()
        assert np.array_equal(got, want[k]), k
    if with_itk:
        assert np.array_equal(d_itk.cpu().numpy(), want["is_token_ids"])
    for g in range(G):
        assert np.array_equal(d_slots[g].cpu().numpy(), want["slot_mappings"][g]), f"group {g}"
        assert np.array_equal(d_tables[g].cpu().numpy(), tables[g]), "table modified"


def test_pages_benchmark_config():
    """Section 11's configuration: position 24576, two KV groups of page 16,
    128 request slots, 4096 token slots, M-RoPE."""
    _run(24576, [16, 16], n_tokens=4096, n_reqs=128, mrope=True)


@pytest.mark.parametrize("position", [0, 1, 783, 784, 831, 832, 8192, 32767])
def test_three_groups_mixed_pages(position):
    _run(position, [16, 784, 832], mrope=True, delta=-37, with_itk=True, seed=position)


def test_single_group_no_mrope():
    _run(8192, [832], n_tokens=8, n_reqs=1)


def test_no_kv_groups():
    _run(12345, [], n_reqs=300)          # arrays longer than one wave's stride


def test_many_groups():
    _run(20000, [16, 32, 64, 128, 784, 832, 1024, 3], seed=3)
