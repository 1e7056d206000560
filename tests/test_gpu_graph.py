"""GPU: the library's launches captured in a HIP graph (through torch's graph
capture) and replayed several times, with eager work and synchronisations
between the replays; every replay must give the eager result bit for bit.
Covers the two-kernel decode with the fused KV write, the prefill chunk with
its split plan (partials in the workspace, then the merge kernel) and the
GEMV."""
import numpy as np
import pytest

import workloads as W
from gpu_util import log, to_dev

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _pa():
    import prefill_block_table_amd as pa
    return pa


def _replay_and_check(run, outs, eager_ref, name):
    """Capture run() (which writes into the preallocated outs), replay it
    REPLAYS times with unrelated eager work in between, and compare."""
    import torch
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    scratch = torch.randn(1 << 20, device="cuda")
    for i in range(REPLAYS):
        for o in outs:
            o.view(torch.int16).fill_(-7)          # poison the outputs between replays
        scratch.mul_(1.0001).add_(float(i))        # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, ref in zip(outs, eager_ref):
            assert torch.equal(o.view(torch.int16), ref.view(torch.int16)), f"{name} replay {i}"
    log(f"{name}: {REPLAYS} replays bit-identical to the eager run")


def test_decode_append_graph_replays():
    import torch
    pa = _pa()
    c = W.decode_8k()
    log(c.name + " graph")
    k, v = to_dev(c.k_cache), to_dev(c.v_cache)
    bt, sl, q = to_dev(c.block_tables), to_dev(c.seq_lens), to_dev(c.q)
    kn, vn = to_dev(c.k_new), to_dev(c.v_new)
    ws = pa.decode_workspace(q.shape[0], c.max_seq_len, c.block_size)
    out = torch.empty_like(q)

    def run():
        pa.decode_append(q, k, v, bt, sl, c.max_seq_len, c.scale, kn, vn, workspace=ws, out=out)

    run()
    torch.cuda.synchronize()
    ref = out.clone()
    _replay_and_check(run, [out], [ref], "decode_append 8K")


def test_prefill_split_plan_graph_replays():
    import torch
    pa = _pa()
    case = W.prefill_8k()
    ch = case.chunks[1]                      # q = 1685: the split plan and the merge kernel
    log(f"prefill q={ch.q_len} graph")
    k, v, bt = to_dev(case.k_cache), to_dev(case.v_cache), to_dev(case.block_table)
    pos = to_dev(np.arange(ch.start_pos, ch.start_pos + ch.q_len, dtype=np.int64))
    pa.kv_write_fused(k, v, to_dev(ch.k_new), to_dev(ch.v_new), pos, bt)
    q = to_dev(ch.q)
    out = torch.empty_like(q)
    ws = pa.prefill_workspace(ch.q_len, ch.start_pos, case.block_size)

    def run():
        pa.prefill_chunk(q, k, v, bt, ch.start_pos, case.scale, causal=True, out=out, workspace=ws)

    run()
    torch.cuda.synchronize()
    ref = out.clone()
    _replay_and_check(run, [out], [ref], f"prefill q={ch.q_len}")


def test_gemv_graph_replays():
    import torch
    pa = _pa()
    Wb, xb = W.make_gemv_case(5, 14336, 5120)
    log("gemv 14336 x 5120 graph")
    Wd, xd = to_dev(Wb), to_dev(xb)
    y = torch.empty(14336, dtype=torch.bfloat16, device="cuda")

    def run():
        pa.gemv(Wd, xd, out=y)

    run()
    torch.cuda.synchronize()
    ref = y.clone()
    _replay_and_check(run, [y], [ref], "gemv")
