"""GPU: the library's launches captured in a HIP graph (through torch's graph
capture) and replayed several times, with eager work and synchronisations
between the replays; every replay must give the eager result bit for bit.
Covers the two-kernel decode with the fused KV write, the prefill chunk with
its split plan (partials in the workspace, then the merge kernel), the
several-sequence prefill, the fused slot-mapping KV write (caches restored
between replays), the separate slot mapping, KV write and plain decode in one
graph, the single-token input preparation and the GEMV."""
import numpy as np
import pytest

import workloads as W
from gpu_util import log, to_dev

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _pa():
    import prefill_block_table_amd as pa
    return pa


def _replay_and_check(run, outs, eager_ref, name, poison=None):
    """Capture run() (which writes into the preallocated outs), replay it
    REPLAYS times with unrelated eager work in between, and compare.
    poison(): restores the pre-call state between replays (default: fill
    the outputs with a pattern no call writes)."""
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
        if poison is None:
            for o in outs:
                o.view(torch.int16).fill_(-7)      # poison the outputs between replays
        else:
            poison()
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


def test_prefill_varlen_graph_replays():
    import torch
    pa = _pa()
    B = 832
    seqs = [(0, 1), (700, 300), (4000, 129), (2496, 64)]
    pages = sum(-(-(s0 + n) // B) for s0, n in seqs)
    c = W.make_varlen_prefill_case("varlen_graph", 85, seqs, B, pages + 4, causal=True)
    log(c.name + " graph")
    k, v, bt = to_dev(c.k_cache), to_dev(c.v_cache), to_dev(c.block_tables)
    for sq, ch in enumerate(c.chunks):
        pos = to_dev(np.arange(ch.start_pos, ch.start_pos + ch.q_len, dtype=np.int64))
        pa.kv_write_fused(k, v, to_dev(ch.k_new), to_dev(ch.v_new), pos, bt,
                          to_dev(np.full(ch.q_len, sq, dtype=np.int32)))
    lens = [ch.q_len for ch in c.chunks]
    cu = to_dev(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32))
    used_np = np.array([ch.start_pos + ch.q_len for ch in c.chunks], dtype=np.int32)
    used = to_dev(used_np)
    q = to_dev(np.concatenate([ch.q for ch in c.chunks]))
    out = torch.empty_like(q)

    def run():
        pa.prefill_varlen(q, k, v, bt, cu, used, max(lens), int(used_np.max()), c.scale,
                          causal=True, out=out)

    run()
    torch.cuda.synchronize()
    ref = out.clone()
    _replay_and_check(run, [out], [ref], "prefill_varlen")


def test_kv_write_fused_graph_replays():
    """The write's destination is the cache itself: between replays the
    caches are put back to their state before the call, so each replay has
    to write the same rows again."""
    import torch
    pa = _pa()
    c = W.decode_8k()
    log("kv_write_fused graph")
    k, v = to_dev(c.k_cache), to_dev(c.v_cache)
    k0, v0 = k.clone(), v.clone()
    bt = to_dev(c.block_tables)
    pos, seq = to_dev(c.positions), to_dev(c.token_seq)
    kn, vn = to_dev(c.k_new), to_dev(c.v_new)
    slots = torch.empty(pos.shape[0], dtype=torch.int64, device="cuda")

    def run():
        pa.kv_write_fused(k, v, kn, vn, pos, bt, seq, slot_out=slots)

    run()
    torch.cuda.synchronize()
    refs = [k.clone(), v.clone(), slots.clone()]
    assert not torch.equal(k.view(torch.int16), k0.view(torch.int16)), "the eager write changed nothing"

    def poison():
        k.copy_(k0)
        v.copy_(v0)
        slots.fill_(-7)

    _replay_and_check(run, [k, v, slots], refs, "kv_write_fused", poison=poison)


def test_decode_input_prep_graph_replays():
    import torch
    pa = _pa()
    log("decode_input_prep graph")
    position, block_sizes, n_tokens, n_reqs = 24576, [16, 16], 4096, 128
    rng = np.random.Generator(np.random.PCG64(11))
    tables = [to_dev(rng.permutation(1 << 20)[: -(-(position + 1) // B) + 2].astype(np.int32))
              for B in block_sizes]
    input_ids = torch.full((n_tokens,), -7, dtype=torch.int32, device="cuda")
    positions = torch.full((3, n_tokens + 1), -7, dtype=torch.int64, device="cuda")
    qsl = torch.full((n_reqs + 1,), -7, dtype=torch.int32, device="cuda")
    seq_lens = torch.full((n_reqs,), -7, dtype=torch.int32, device="cuda")
    discard = torch.ones(n_reqs, dtype=torch.uint8, device="cuda")
    slots = [torch.full((n_tokens,), -7, dtype=torch.int64, device="cuda") for _ in block_sizes]
    sampled = to_dev(np.array([151_643, 99], np.int64))
    bsz = to_dev(np.array(block_sizes, np.int32))
    btp = torch.tensor([t.data_ptr() for t in tables], dtype=torch.int64, device="cuda")
    smp = torch.tensor([s.data_ptr() for s in slots], dtype=torch.int64, device="cuda")
    outs = [input_ids, positions, qsl, seq_lens, discard] + slots

    def run():
        pa.decode_input_prep(sampled, position, input_ids, positions, qsl, seq_lens, discard,
                             block_sizes=bsz, block_table_ptrs=btp, slot_mapping_ptrs=smp,
                             mrope=True, mrope_delta=-37)

    run()
    torch.cuda.synchronize()
    refs = [o.clone() for o in outs]

    def poison():
        for o in outs:
            o.fill_(-7 if o.dtype != torch.uint8 else 3)

    _replay_and_check(run, outs, refs, "decode_input_prep", poison=poison)


def test_slot_mapping_kv_write_and_decode_graph_replays():
    """The separate calls in one graph: pa_slot_mapping, pa_kv_write through
    those slots, then the plain pa_decode (caches restored between replays)."""
    import torch
    pa = _pa()
    c = W.batched_decode()
    log("slot_mapping + kv_write + decode graph")
    k, v = to_dev(c.k_cache), to_dev(c.v_cache)
    k0, v0 = k.clone(), v.clone()
    bt, sl, q = to_dev(c.block_tables), to_dev(c.seq_lens), to_dev(c.q)
    pos, seq = to_dev(c.positions), to_dev(c.token_seq)
    kn, vn = to_dev(c.k_new), to_dev(c.v_new)
    ws = pa.decode_workspace(q.shape[0], c.max_seq_len, c.block_size)
    slots = torch.empty(pos.shape[0], dtype=torch.int64, device="cuda")
    out = torch.empty_like(q)

    def run():
        pa.slot_mapping(pos, bt, c.block_size, token_seq=seq, out=slots)
        pa.kv_write(k, v, kn, vn, slots)
        pa.decode(q, k, v, bt, sl, c.max_seq_len, c.scale, workspace=ws, out=out)

    run()
    torch.cuda.synchronize()
    refs = [k.clone(), v.clone(), slots.clone(), out.clone()]

    def poison():
        k.copy_(k0)
        v.copy_(v0)
        slots.fill_(-7)
        out.view(torch.int16).fill_(-7)

    _replay_and_check(run, [k, v, slots, out], refs, "slot_mapping + kv_write + decode", poison=poison)
