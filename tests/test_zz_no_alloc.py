"""GPU: the allocation-free decode entry point (pa_decode_noalloc, called
through the C ABI with ctypes) against pa_decode with a caller workspace:
two calls in a row, the second with a smaller batch, each output identical
bit for bit to pa_decode's (the same kernels) and within the oracle
tolerance; a batch beyond the static scratch is rejected on the host; the
call captured in a HIP graph replays bit-identically to the eager call."""
import ctypes

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import bits, compare, log, to_dev

pytestmark = pytest.mark.gpu


def _noalloc(pa, case, q, k, v, bt, sl, out):
    """One pa_decode_noalloc call on the current stream (q, k, v, bt, sl, out
    already on the device: nothing is copied, so the call can be captured)."""
    import torch
    S = case.q.shape[0]
    rc = pa.lib.pa_decode_noalloc(
        ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
        ctypes.c_void_p(v.data_ptr()), k.stride(0), ctypes.c_void_p(bt.data_ptr()), bt.shape[1],
        ctypes.c_void_p(sl.data_ptr()), S, case.max_seq_len, case.block_size, case.scale, 24, 4, 256,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, pa.strerror(rc)


def _written(case):
    k, v = case.k_cache, case.v_cache
    if len(case.positions):
        slots = oracle.slot_mapping(case.positions, case.token_seq, case.block_tables, case.block_size)
        k, v = oracle.kv_write(k, v, case.k_new, case.v_new, slots)
    return k, v


def test_noalloc_matches_workspace_decode_two_calls():
    import torch
    import prefill_block_table_amd as pa
    big = W.batched_decode(seed=61)               # 16 sequences, 4K-32K tokens
    small = W.decode_8k(seed=62)                  # 1 sequence, 8193 tokens
    outs = []
    for case in (big, small):
        kh, vh = _written(case)
        k, v = to_dev(kh), to_dev(vh)
        bt, sl = to_dev(case.block_tables), to_dev(case.seq_lens)
        log(f"noalloc {case.name} seqs={case.q.shape[0]} max_seq_len={case.max_seq_len}")
        out_na = torch.full(case.q.shape, 0x7FC0, dtype=torch.int16, device="cuda").view(torch.bfloat16)
        q = to_dev(case.q)
        _noalloc(pa, case, q, k, v, bt, sl, out_na)
        ref_out = pa.decode(q, k, v, bt, sl, case.max_seq_len, case.scale)
        torch.cuda.synchronize()
        a, b = bits(out_na), bits(ref_out)
        assert np.array_equal(a, b), f"{case.name}: pa_decode_noalloc differs from pa_decode"
        outs.append(a)
        compare(a, oracle.decode(case.q, kh, vh, case.block_tables, case.seq_lens, case.block_size,
                                 case.scale), case.name + " noalloc")
    # the second (smaller) call left the first call's results alone
    assert outs[0].shape[0] == 16 and outs[1].shape[0] == 1


def test_noalloc_rejects_batches_beyond_the_scratch():
    import prefill_block_table_amd as pa
    FAKE = ctypes.c_void_p(0x10000)
    need = pa.decode_workspace_size(4000, 1000, 64, 4)
    assert need > (16 << 20)
    rc = pa.lib.pa_decode_noalloc(FAKE, FAKE, FAKE, FAKE, 64 * 1024, FAKE, 16, FAKE, 4000, 1000, 64,
                                  0.0625, 24, 4, 256, None)
    assert rc == -11 and "scratch" in pa.strerror(rc)


def test_noalloc_graph_replays():
    """pa_decode_noalloc captured in a HIP graph (its scratch is a fixed device
    address, so the captured launches stay valid): every replay, with other
    eager work and a poisoned output between replays, equals the eager call."""
    import torch
    import prefill_block_table_amd as pa
    case = W.decode_8k(seed=63)
    kh, vh = _written(case)
    k, v = to_dev(kh), to_dev(vh)
    bt, sl = to_dev(case.block_tables), to_dev(case.seq_lens)
    q = to_dev(case.q)
    out = torch.empty(case.q.shape, dtype=torch.bfloat16, device="cuda")
    log(f"noalloc graph {case.name}")
    _noalloc(pa, case, q, k, v, bt, sl, out)       # eager call first (sets up the scratch address)
    torch.cuda.synchronize()
    ref = out.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            _noalloc(pa, case, q, k, v, bt, sl, out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    other = torch.randn(1 << 20, device="cuda")
    for i in range(4):
        out.view(torch.int16).fill_(-7)
        other.mul_(1.0001).add_(float(i))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"replay {i}"
    log("noalloc graph: 4 replays bit-identical to the eager call")
