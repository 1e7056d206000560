#!/usr/bin/env python3
"""Benchmark of the paged-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step = one decode step of the 8K-context workload: the slot-mapping
KV-cache write of the new token (position 8192) and the split-K decode over
its 8193 keys (page 832, 24 query / 4 KV heads, head 256, bf16), issued as one
pa_decode_append call (the write happens inside the decode launch).  `value` is decode K/V bytes moved per second over the whole timed
region (K/V bytes = seq_len * 4 heads * 256 * 2 B * 2 for K and V); each step
reads a different replica of the KV pool so that the reads come from HBM,
not from the 256 MB Infinity Cache.  The same run also measures the other
figures the metric names (decode at 32K context for pages 784/832/1024, the
16-sequence batch, and the q=4096 / q=1685 prefill chunks in TFLOP/s), which
are reported under "extra".  Prints one JSON line.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor spec
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_ctx8192_b832_hbm_traffic.json")
DECODE_SRC = os.path.join(ROOT, "prefill_block_table_amd", "csrc", "decode.hip")
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, vendor spec
MALL_DEFEAT_BYTES = 2 << 30    # rotate pool replicas so that the K/V bytes the steps
                               # touch cycle over at least this many bytes (8x the
                               # 256 MB Infinity Cache)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-extra", action="store_true", help="headline workload only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--prefill-pass", action="store_true",
                    help="for rocprofv3 --pmc runs: 5 launches of each prefill chunk")
    ap.add_argument("--gemv-pass", action="store_true",
                    help="only the GEMV leg and a calibration copy (for rocprofv3 runs)")
    ap.add_argument("--counter-pass", action="store_true",
                    help="for rocprofv3 --pmc runs: a few headline decode steps, then a "
                         "256 MiB device-to-device copy that calibrates FETCH_SIZE/WRITE_SIZE")
    return ap.parse_args()


def kv_bytes(seq_lens, num_kv_heads=4):
    return int(sum(int(x) for x in seq_lens)) * num_kv_heads * 256 * 2 * 2


SERVING_BATCHES = ((512, 256), (256, 1024), (128, 512), (64, 2048))


def bench_decode_serving(D, pa, steps=100, warmup=10, block_size=64):
    """Serving-style decode batches: S sequences of L cached tokens each plus
    the appended one, 24 / 4 heads, page 64, random page placement; the
    caches are drawn on the device (seeded) and rotated over >= 2 GiB of
    replicas as in the other decode legs.  Returns per-batch timings."""
    torch = D.torch
    res = {}
    for S, L in SERVING_BATCHES:
        g = torch.Generator(device=D.dev).manual_seed(1000 * S + L)
        per = -(-(L + 1) // block_size)
        P = S * per + 1
        k0 = torch.randn(P, block_size, 4, 256, device=D.dev, generator=g).to(torch.bfloat16)
        v0 = torch.randn(P, block_size, 4, 256, device=D.dev, generator=g).to(torch.bfloat16)
        reps = max(1, math.ceil(MALL_DEFEAT_BYTES / (2 * k0.numel() * 2)))
        ks, vs = [k0], [v0]
        for _ in range(reps - 1):
            ks.append(k0.clone())
            vs.append(v0.clone())
        bt = torch.randperm(P - 1, device=D.dev, generator=g)[: S * per].view(S, per).to(torch.int32)
        sl = torch.full((S,), L + 1, dtype=torch.int32, device=D.dev)
        q = torch.randn(S, 24, 256, device=D.dev, generator=g).to(torch.bfloat16)
        kn = torch.randn(S, 4, 256, device=D.dev, generator=g).to(torch.bfloat16)
        vn = torch.randn(S, 4, 256, device=D.dev, generator=g).to(torch.bfloat16)
        ws = pa.decode_workspace(S, L + 1, block_size, device=D.dev)
        out = torch.empty_like(q)
        for i in range(warmup):
            pa.decode_append(q, ks[i % reps], vs[i % reps], bt, sl, L + 1, 0.0625, kn, vn, workspace=ws, out=out)
        torch.cuda.synchronize()
        torch.cuda._sleep(int(50e6))               # let the host enqueue ahead of the device
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(steps):
            pa.decode_append(q, ks[i % reps], vs[i % reps], bt, sl, L + 1, 0.0625, kn, vn, workspace=ws, out=out)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        nbytes = S * (L + 1) * 4 * 256 * 2 * 2
        res[f"{S}x{L}"] = {"ms_per_step": ms, "kv_bytes": nbytes, "gbs": nbytes / (ms * 1e-3) / 1e9,
                           "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "replicas": reps}
        del ks, vs, k0, v0
        torch.cuda.empty_cache()
    return res


def causal_flops(start, q_len, num_q_heads=24, head_dim=256):
    pairs = q_len * start + q_len * (q_len + 1) // 2
    return 4 * head_dim * num_q_heads * pairs


class Dev:
    def __init__(self):
        import numpy as np
        import torch
        self.np, self.torch = np, torch
        self.dev = torch.device("cuda:0")

    def t(self, a):
        a = self.np.ascontiguousarray(a)
        if a.dtype == self.np.uint16:
            return self.torch.from_numpy(a.view(self.np.int16)).to(self.dev).view(self.torch.bfloat16)
        return self.torch.from_numpy(a).to(self.dev)


_SLEEP_CYCLES_PER_MS = None


def gpu_hold(torch, ms):
    """Keep the GPU busy for about `ms` so the host can enqueue the timed steps
    ahead of the device; the timed region then measures device execution, not
    Python launch overhead.  Not part of any timed region."""
    global _SLEEP_CYCLES_PER_MS
    if _SLEEP_CYCLES_PER_MS is None:
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        torch.cuda._sleep(2_000_000)
        b.record()
        torch.cuda.synchronize()
        _SLEEP_CYCLES_PER_MS = 2_000_000 / max(a.elapsed_time(b), 1e-3)
    torch.cuda._sleep(int(_SLEEP_CYCLES_PER_MS * ms))


def timed_loop(torch, steps, launch_step, hold_ms, events=True):
    """Run `steps` steps after a GPU hold; returns (total_ms, per-step kernel
    ms of the bracketed launch (empty without events), host enqueue seconds)."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           if events else None for _ in range(steps)]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    gpu_hold(torch, hold_ms)
    t0 = time.perf_counter()
    e0.record()
    for i in range(steps):
        launch_step(i, evs[i])
    e1.record()
    host_s = time.perf_counter() - t0
    torch.cuda.synchronize()
    return e0.elapsed_time(e1), ([a.elapsed_time(b) for a, b in evs] if events else []), host_s


def _stats(ts):
    t = sorted(ts)
    return {"kernel_ms_avg": sum(t) / len(t), "kernel_ms_p10": t[len(t) // 10],
            "kernel_ms_p50": t[len(t) // 2], "kernel_ms_p90": t[(9 * len(t)) // 10]}


def bench_decode(D, pa, case, steps, warmup, rotate=True, graph=False, hold_ms=None,
                 separate=False):
    """Timed decode steps (KV write of the new token + decode); returns a dict.
    A step is one decode_append call, or with `separate` a kv_write_fused call
    followed by a decode call."""
    torch = D.torch
    k0, v0 = D.t(case.k_cache), D.t(case.v_cache)
    # replicas sized by the bytes a step touches (not the pool's size), so
    # the rotation cycles over >= MALL_DEFEAT_BYTES of K/V that steps read
    touched = kv_bytes(case.seq_lens)
    reps = max(2, math.ceil(MALL_DEFEAT_BYTES / touched)) if rotate else 1
    ks, vs = [k0], [v0]
    for _ in range(reps - 1):
        ks.append(k0.clone())
        vs.append(v0.clone())
    bt, sl = D.t(case.block_tables), D.t(case.seq_lens)
    q = D.t(case.q)
    has_write = len(case.positions) > 0
    if has_write:
        kn, vn = D.t(case.k_new), D.t(case.v_new)
        pos, seq = D.t(case.positions), D.t(case.token_seq)
    ws = pa.decode_workspace(q.shape[0], case.max_seq_len, case.block_size, device=D.dev)
    out = torch.empty_like(q)

    def step(i, ev=None):
        r = i % reps
        if has_write and not separate:
            pa.decode_append(q, ks[r], vs[r], bt, sl, case.max_seq_len, case.scale, kn, vn,
                             workspace=ws, out=out)
            return
        if has_write:
            pa.kv_write_fused(ks[r], vs[r], kn, vn, pos, bt, seq)
        pa.decode(q, ks[r], vs[r], bt, sl, case.max_seq_len, case.scale, workspace=ws, out=out)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    res = {"replicas": reps, "rotated_kv_bytes": reps * touched if rotate else touched}
    nbytes = kv_bytes(case.seq_lens)
    if graph:
        # one graph holds one step per replica; replayed until >= steps steps ran
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                for i in range(reps):
                    step(i)
        torch.cuda.current_stream().wait_stream(s)
        n_rep = max(1, -(-steps // reps))
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n_rep):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / (n_rep * reps)
        res.update(ms_per_step=ms, steps=n_rep * reps, gbs=nbytes / (ms * 1e-3) / 1e9)
        return res
    hold = hold_ms if hold_ms is not None else 0.25 * steps + 20
    # 1) whole steps, nothing between the launches
    total_ms, _, host_s = timed_loop(torch, steps, lambda i, ev: step(i), hold, events=False)
    # 2) the decode call alone (split + merge kernels), bracketed by events
    def dec_only(i, ev):
        r = i % reps
        ev[0].record()
        if has_write and not separate:
            pa.decode_append(q, ks[r], vs[r], bt, sl, case.max_seq_len, case.scale, kn, vn,
                             workspace=ws, out=out)
        else:
            pa.decode(q, ks[r], vs[r], bt, sl, case.max_seq_len, case.scale, workspace=ws,
                      out=out)
        ev[1].record()
    _, kern, host_k = timed_loop(torch, steps, dec_only, hold)
    st = _stats(kern)
    res.update(call="decode_append" if has_write and not separate else
               ("kv_write_fused + decode" if has_write else "decode"),
               ms_per_step=total_ms / steps, kv_bytes=nbytes,
               gbs=nbytes / (total_ms / steps * 1e-3) / 1e9,
               kernel_gbs=nbytes / (st["kernel_ms_avg"] * 1e-3) / 1e9,
               host_enqueue_ms=host_s * 1e3, hold_ms=hold,
               host_bound=bool(max(host_s, host_k) * 1e3 > hold), **st)
    return res


def bench_prefill(D, pa, case, steps, warmup):
    """Per chunk: the chunk's KV write, then timed attention steps."""
    torch = D.torch
    np = D.np
    k, v = D.t(case.k_cache), D.t(case.v_cache)
    bt = D.t(case.block_table)
    out = {}
    for ch in case.chunks:
        pos = D.t(np.arange(ch.start_pos, ch.start_pos + ch.q_len, dtype=np.int64))
        kn, vn, q = D.t(ch.k_new), D.t(ch.v_new), D.t(ch.q)
        o = torch.empty_like(q)
        ws = pa.prefill_workspace(ch.q_len, ch.start_pos, case.block_size, device=D.dev)
        torch.cuda.synchronize()
        w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        w0.record()
        pa.kv_write_fused(k, v, kn, vn, pos, bt)
        w1.record()
        for _ in range(warmup):
            pa.prefill_chunk(q, k, v, bt, ch.start_pos, case.scale, causal=True, out=o, workspace=ws)

        def step(i, ev):
            if ev is not None:
                ev[0].record()
            pa.prefill_chunk(q, k, v, bt, ch.start_pos, case.scale, causal=True, out=o, workspace=ws)
            if ev is not None:
                ev[1].record()

        # device time per launch of back-to-back launches (the figure), then
        # per-launch event brackets for the spread
        hold = 2.0 * steps + 5.0
        total_ms, _, _ = timed_loop(torch, steps, step, hold, events=False)
        _, kern, _ = timed_loop(torch, steps, step, hold)
        st = _stats(kern)
        avg = total_ms / steps
        fl = causal_flops(ch.start_pos, ch.q_len)
        out[f"q{ch.q_len}_start{ch.start_pos}"] = dict(
            st, ms_per_launch=avg, causal_flops=fl, tflops=fl / (avg * 1e-3) / 1e12,
            frac_bf16_peak=fl / (avg * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
            kv_write_ms=w0.elapsed_time(w1), kv_write_bytes=ch.q_len * 4 * 256 * 2 * 2)
    return out


VARLEN_SEED = 808


def varlen_batch():
    """8 sequences, each one chunk of 256-4096 query rows at a start position in
    [0, 8192] (seeded), page 832: a batched chunked-prefill step."""
    import numpy as np
    rng = np.random.Generator(np.random.PCG64(VARLEN_SEED))
    q_lens = rng.integers(256, 4096, size=8, endpoint=True)
    starts = rng.integers(0, 8192, size=8, endpoint=True)
    return [(int(s0), int(n)) for s0, n in zip(starts, q_lens)]


def bench_prefill_varlen(D, pa, W, steps, warmup, block_size=832):
    """pa_prefill_varlen on the 8-sequence batch above: every sequence's chunk
    K/V written first, then back-to-back launches; TFLOP/s over the causal
    flops of all sequences."""
    torch = D.torch
    np = D.np
    seqs = varlen_batch()
    pages = sum(-(-(s0 + n) // block_size) for s0, n in seqs)
    c = W.make_varlen_prefill_case("varlen8", VARLEN_SEED, seqs, block_size, pages + 4)
    k, v = D.t(c.k_cache), D.t(c.v_cache)
    bt = D.t(c.block_tables)
    for s, ch in enumerate(c.chunks):
        pos = D.t(np.arange(ch.start_pos, ch.start_pos + ch.q_len, dtype=np.int64))
        seq = D.t(np.full(ch.q_len, s, dtype=np.int32))
        pa.kv_write_fused(k, v, D.t(ch.k_new), D.t(ch.v_new), pos, bt, seq)
    lens = [ch.q_len for ch in c.chunks]
    cu = D.t(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32))
    used_np = np.array([ch.start_pos + ch.q_len for ch in c.chunks], dtype=np.int32)
    used = D.t(used_np)
    q = D.t(np.concatenate([ch.q for ch in c.chunks]))
    o = torch.empty_like(q)
    ws = pa.prefill_varlen_workspace(cu, used, max(lens), int(used_np.max()), block_size,
                                     device=D.dev) if hasattr(pa, "prefill_varlen_workspace") else None

    def step(i, ev):
        if ev is not None:
            ev[0].record()
        if ws is None:
            pa.prefill_varlen(q, k, v, bt, cu, used, max(lens), int(used_np.max()), c.scale,
                              causal=True, out=o)
        else:
            pa.prefill_varlen(q, k, v, bt, cu, used, max(lens), int(used_np.max()), c.scale,
                              causal=True, out=o, workspace=ws)
        if ev is not None:
            ev[1].record()

    for i in range(warmup):
        step(i, None)
    hold = 2.0 * steps + 5.0
    total_ms, _, _ = timed_loop(torch, steps, step, hold, events=False)
    _, kern, _ = timed_loop(torch, steps, step, hold)
    avg = total_ms / steps
    fl = sum(causal_flops(s0, n) for s0, n in seqs)
    return dict(_stats(kern), seqs=[{"start": s0, "q_len": n} for s0, n in seqs],
                block_size=block_size, ms_per_launch=avg, causal_flops=fl,
                tflops=fl / (avg * 1e-3) / 1e12,
                frac_bf16_peak=fl / (avg * 1e-3) / 1e12 / BF16_PEAK_TFLOPS)


def bench_input_prep(D, pa, iters=2000, warmup=100):
    """Single-token decode input preparation at the input-prep post's
    benchmark configuration (position 24576, two KV groups of page 16, 128
    request slots, 4096 token slots, M-RoPE): device time per launch of
    back-to-back launches, and host time per call through the binding."""
    torch = D.torch
    np = D.np
    P, R, N, Bs = 24576, 128, 4096, [16, 16]
    dev = "cuda"
    sampled = torch.tensor([151_643], dtype=torch.int64, device=dev)
    ids = torch.zeros(N, dtype=torch.int32, device=dev)
    pos = torch.zeros(3, N + 1, dtype=torch.int64, device=dev)
    qsl = torch.zeros(R + 1, dtype=torch.int32, device=dev)
    sl = torch.zeros(R, dtype=torch.int32, device=dev)
    mask = torch.ones(R, dtype=torch.bool, device=dev)
    rng = np.random.Generator(np.random.PCG64(24576))
    tables = [torch.from_numpy(rng.permutation(1 << 16)[:2048].astype(np.int32)).to(dev) for _ in Bs]
    slots = [torch.zeros(N, dtype=torch.int64, device=dev) for _ in Bs]
    bs = torch.tensor(Bs, dtype=torch.int32, device=dev)
    btp = torch.tensor([t.data_ptr() for t in tables], dtype=torch.int64, device=dev)
    smp = torch.tensor([t.data_ptr() for t in slots], dtype=torch.int64, device=dev)

    def step(i, ev=None):
        pa.decode_input_prep(sampled, P, ids, pos, qsl, sl, mask, block_sizes=bs,
                             block_table_ptrs=btp, slot_mapping_ptrs=smp, mrope=True)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    total_ms, _, host_s = timed_loop(torch, iters, step, 0.02 * iters + 20, events=False)
    return {"config": "position 24576, 2 KV groups of page 16, 128 request slots, 4096 token "
                      "slots, M-RoPE", "launches": iters,
            "device_us_per_launch": total_ms / iters * 1e3,
            "host_us_per_call": host_s / iters * 1e6}


def bench_gemv(D, pa, W, iters=40, warmup=10, rotate_bytes=1 << 30):
    """Decode-time bf16 M=1 linear layer y = W x at the measurement post's
    three weight shapes (warmup 10, 40 timed launches, as there).  Each timed
    launch reads a different copy of the weights, cycling over at least 1 GiB
    of copies, so no launch finds its weights in the 256 MB last-level cache,
    as in a decode step where every layer has its own weights.  Reports the
    kernel's average launch time (HIP events around each launch) and its
    weight bandwidth, and torch.mv (the vendor BLAS) under the same rotation."""
    torch = D.torch
    out = {}
    for N, K in W.GEMV_SHAPES:
        g = torch.Generator(device=D.dev)
        g.manual_seed(N)
        w_bytes = N * K * 2
        copies = max(2, -(-rotate_bytes // w_bytes))
        Ws = [(torch.randn(N, K, generator=g, device=D.dev) * 0.02).to(torch.bfloat16)
              for _ in range(copies)]
        x = torch.randn(K, generator=g, device=D.dev).to(torch.bfloat16)
        y = torch.empty(N, dtype=torch.bfloat16, device=D.dev)
        res = {}
        for name, fn in (("pa_gemv_bf16", lambda w: pa.gemv(w, x, out=y)),
                         ("torch_mv", lambda w: torch.mv(w, x))):
            def step(i, ev=None, fn=fn):
                if ev is not None:
                    ev[0].record()
                fn(Ws[i % copies])
                if ev is not None:
                    ev[1].record()
            for i in range(warmup):
                step(i)
            torch.cuda.synchronize()
            _, ts, _ = timed_loop(torch, iters, step, 0.3 * iters + 5)
            st = _stats(ts)
            res[name] = {"kernel_ms_avg": round(st["kernel_ms_avg"], 6),
                         "kernel_ms_p50": round(st["kernel_ms_p50"], 6),
                         "weight_gbs": round(w_bytes / (st["kernel_ms_avg"] * 1e-3) / 1e9, 1)}
        gbs = res["pa_gemv_bf16"]["weight_gbs"]
        res["hbm_frac"] = round(gbs / HBM_PEAK_GBS, 4)
        res["weight_copies"] = copies
        res["algorithmic_bytes_per_launch"] = w_bytes + 2 * K + 2 * N
        out[f"{N}x{K}"] = res
        del Ws
        torch.cuda.empty_cache()
    return out


def decode_src_sha():
    import hashlib
    with open(DECODE_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic():
    """HBM bytes per pa_decode launch from the committed counter runs, or None
    when the decode kernels changed since those counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("decode_src_sha") != decode_src_sha():
        return None
    return t.get("hbm_bytes_per_launch")


def counter_pass(D, pa, W):
    """Launch sequence profiled by the --pmc runs: 10 headline decode steps on
    distinct pool replicas, then a plain 256 MiB copy of known size."""
    torch = D.torch
    case = W.decode_8k()
    k0, v0 = D.t(case.k_cache), D.t(case.v_cache)
    bt, sl, q = D.t(case.block_tables), D.t(case.seq_lens), D.t(case.q)
    kn, vn = D.t(case.k_new), D.t(case.v_new)
    ws = pa.decode_workspace(1, case.max_seq_len, case.block_size, device=D.dev)
    out = torch.empty_like(q)
    for _ in range(10):
        k, v = k0.clone(), v0.clone()           # fresh replica: cold in L2 and MALL
        torch.cuda.synchronize()
        pa.decode_append(q, k, v, bt, sl, case.max_seq_len, case.scale, kn, vn, workspace=ws,
                         out=out)
        torch.cuda.synchronize()
    src = torch.empty(256 << 20, dtype=torch.uint8, device=D.dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()


def gemv_pass(D, pa, W):
    """Launch sequence profiled for the GEMV summaries: the GEMV leg (three
    weight shapes, the library kernel and torch.mv), then a plain 256 MiB copy
    of known size that calibrates the HBM byte counters."""
    torch = D.torch
    print(json.dumps({"gemv_bf16_m1": bench_gemv(D, pa, W)}), flush=True)
    src = torch.empty(256 << 20, dtype=torch.uint8, device=D.dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()


def prefill_pass(D, pa, W):
    """Launch sequence profiled by the prefill --pmc runs: per chunk of the
    8K prefill workload, the chunk's KV write, then 5 attention launches."""
    torch = D.torch
    np = D.np
    case = W.prefill_8k()
    k, v, bt = D.t(case.k_cache), D.t(case.v_cache), D.t(case.block_table)
    for ch in case.chunks:
        pos = D.t(np.arange(ch.start_pos, ch.start_pos + ch.q_len, dtype=np.int64))
        pa.kv_write_fused(k, v, D.t(ch.k_new), D.t(ch.v_new), pos, bt)
        q = D.t(ch.q)
        o = torch.empty_like(q)
        ws = pa.prefill_workspace(ch.q_len, ch.start_pos, case.block_size, device=D.dev)
        for _ in range(5):
            pa.prefill_chunk(q, k, v, bt, ch.start_pos, case.scale, causal=True, out=o, workspace=ws)
        torch.cuda.synchronize()


def cpu_baseline(case, seconds):
    """The fp64 oracle on the headline workload, repeated for ~`seconds`."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count()
    slots = oracle.slot_mapping(case.positions, case.token_seq, case.block_tables, case.block_size)
    n, t0 = 0, time.perf_counter()
    while True:
        k, v = oracle.kv_write(case.k_cache, case.v_cache, case.k_new, case.v_new, slots)
        oracle.decode(case.q, k, v, case.block_tables, case.seq_lens, case.block_size, case.scale)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds or n >= 1000:
            break
    nbytes = kv_bytes(case.seq_lens) * n
    return {"value": nbytes / el / 1e9, "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n} full decode steps (KV write + decode) of the 8K-context workload, "
                      f"{el:.1f} s on the host CPU (fp64 NumPy oracle)"}


def oracle_timings(W):
    """The fp64 oracle on the other workloads, beside the GPU figures: one
    32K-context decode step (page 832), one step of the 16-sequence batch
    (timed on four of its sequences, scaled by K/V bytes), and
    each prefill chunk on a sample of 256 query rows spread over the chunk,
    scaled to the whole chunk by rows (a row's cost grows with its causal key
    count; the sample's rows are evenly spaced, so their mean cost is the
    chunk's).  Milliseconds of host time."""
    import numpy as np
    import oracle
    out = {}
    for name, case, sample in (("decode_ctx32768_b832", W.decode_32k(832), None),
                               ("decode_batch16_ctx4k_32k_b832", W.batched_decode(), [0, 1, 2, 3])):
        k, v = case.k_cache, case.v_cache
        if len(case.positions):
            slots = oracle.slot_mapping(case.positions, case.token_seq, case.block_tables,
                                        case.block_size)
            k, v = oracle.kv_write(k, v, case.k_new, case.v_new, slots)
        t0 = time.perf_counter()
        oracle.decode(case.q, k, v, case.block_tables, case.seq_lens, case.block_size, case.scale,
                      seqs=sample)
        el = time.perf_counter() - t0
        if sample is None:
            out[name] = {"ms_per_step": round(el * 1e3, 1)}
        else:
            frac = kv_bytes(case.seq_lens[sample]) / kv_bytes(case.seq_lens)
            out[name] = {"ms_per_step_est": round(el * 1e3 / frac, 1),
                         "sample": f"sequences {sample} ({el * 1e3:.1f} ms, {frac:.3f} of the "
                                   f"K/V bytes), scaled by K/V bytes"}
    case = W.prefill_8k()
    for ch in case.chunks:
        pos = np.arange(ch.start_pos, ch.start_pos + ch.q_len, dtype=np.int64)
        slots = oracle.slot_mapping(pos, None, case.block_table, case.block_size)
        k, v = oracle.kv_write(case.k_cache, case.v_cache, ch.k_new, ch.v_new, slots)
        rows = np.linspace(0, ch.q_len - 1, min(256, ch.q_len)).astype(np.int64)
        K = oracle.gather_kv(k, case.block_table, ch.start_pos + ch.q_len, case.block_size)
        V = oracle.gather_kv(v, case.block_table, ch.start_pos + ch.q_len, case.block_size)
        t0 = time.perf_counter()
        oracle.attend(ch.q[rows], ch.start_pos + rows, K, V, case.scale, causal=True)
        el = time.perf_counter() - t0
        out[f"prefill_q{ch.q_len}_start{ch.start_pos}"] = {
            "ms_per_chunk_est": round(el * 1e3 * ch.q_len / len(rows), 1),
            "sample": f"{len(rows)} of {ch.q_len} rows ({el * 1e3:.1f} ms), scaled by rows"}
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(multi-GPU sharding is not built).", file=sys.stderr)
        sys.exit(2)
    import torch
    import prefill_block_table_amd as pa
    import workloads as W
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    D = Dev()
    print(f"[bench] {pa.build_info()}", file=sys.stderr, flush=True)
    if args.counter_pass:
        counter_pass(D, pa, W)
        return
    if args.prefill_pass:
        prefill_pass(D, pa, W)
        return
    if args.gemv_pass:
        gemv_pass(D, pa, W)
        return

    head_case = W.decode_8k()
    print("[bench] decode_ctx8192_b832 rotated", file=sys.stderr, flush=True)
    head = bench_decode(D, pa, head_case, args.steps, args.warmup, rotate=True)
    extra = {"decode_ctx8192_b832": head}
    if not args.no_extra:
        print("[bench] decode_ctx8192_b832 warm / graph", file=sys.stderr, flush=True)
        extra["decode_ctx8192_b832_warm"] = bench_decode(D, pa, head_case, args.steps, args.warmup,
                                                         rotate=False)
        extra["decode_ctx8192_b832_graph"] = bench_decode(D, pa, head_case, args.steps,
                                                          args.warmup, rotate=True, graph=True)
        extra["decode_ctx8192_b832_separate_write"] = bench_decode(
            D, pa, head_case, args.steps, args.warmup, rotate=True, separate=True)
        for B in (784, 832, 1024):
            print(f"[bench] decode_ctx32768_b{B}", file=sys.stderr, flush=True)
            extra[f"decode_ctx32768_b{B}"] = bench_decode(D, pa, W.decode_32k(B), args.steps,
                                                          args.warmup, rotate=True)
        print("[bench] decode_batch16", file=sys.stderr, flush=True)
        extra["decode_batch16_ctx4k_32k_b832"] = bench_decode(D, pa, W.batched_decode(),
                                                              max(20, args.steps // 4),
                                                              args.warmup, rotate=True)
        print("[bench] decode serving batches", file=sys.stderr, flush=True)
        extra["decode_serving_b64"] = bench_decode_serving(D, pa)
        print("[bench] decode input prep", file=sys.stderr, flush=True)
        extra["decode_input_prep"] = bench_input_prep(D, pa)
        print("[bench] gemv", file=sys.stderr, flush=True)
        extra["gemv_bf16_m1"] = bench_gemv(D, pa, W)
        print("[bench] prefill", file=sys.stderr, flush=True)
        extra["prefill_b832"] = bench_prefill(D, pa, W.prefill_8k(), max(10, args.steps // 5),
                                              min(args.warmup, 5))
        for B in (784, 1024):
            # the same chunks on the other page sizes (same causal flops)
            print(f"[bench] prefill page {B}", file=sys.stderr, flush=True)
            extra[f"prefill_b{B}"] = bench_prefill(
                D, pa, W.make_prefill_case(f"prefill_q4096_s4096_then_q1685_b{B}", 3,
                                           [(4096, 4096), (8192, 1685)], B, 128),
                max(10, args.steps // 5), min(args.warmup, 5))
        for key in ("q4096_start4096", "q1685_start8192"):
            base = extra["prefill_b832"][key]["ms_per_launch"]
            for B in (784, 1024):
                extra[f"prefill_b{B}"][key]["ratio_to_b832"] = round(
                    extra[f"prefill_b{B}"][key]["ms_per_launch"] / base, 4)
        print("[bench] prefill varlen", file=sys.stderr, flush=True)
        extra["prefill_varlen8_b832"] = bench_prefill_varlen(D, pa, W, max(10, args.steps // 5),
                                                             min(args.warmup, 5))
    torch.cuda.synchronize()

    cpu = None
    if not args.no_cpu:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(head_case, args.cpu_seconds)
        if not args.no_extra:
            print("[bench] oracle on the other workloads", file=sys.stderr, flush=True)
            extra["oracle_ms"] = oracle_timings(W)

    # the launch's average duration over the timed region: HIP events before
    # and after the K back-to-back calls, divided by K (one call per step)
    achieved = head["gbs"]
    line = {
        "metric": "decode K/V GB/s (% HBM peak) @8K/32K ctx; prefill q=4096 TFLOP/s (% MFMA)",
        "value": round(head["gbs"], 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 K/V/q, random block tables)",
        "config": {"workload": "decode_ctx8192_b832: 1 seq, 8192 cached tokens + 1 written at "
                               "position 8192 (slot-mapping KV write inside the split-K decode "
                               "launch), page 832, "
                               "pool 64 pages, 24 q / 4 KV heads, head_dim 256",
                   "kv_bytes_per_step": head["kv_bytes"], "pool_replicas": head["replicas"]},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 3), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(),
                     "kernel": "pa_decode_append (decode_split_kernel + decode_merge_kernel)",
                     "launch_ms_avg": round(head["ms_per_step"], 6),
                     "launch_ms_avg_source": "HIP events around the K timed calls on their "
                                             "stream, divided by K",
                     "algorithmic_bytes_per_launch": head["kv_bytes"],
                     # each call bracketed by its own pair of events (the two event
                     # records between calls add their own time)
                     "launch_ms_avg_bracketed": round(head["kernel_ms_avg"], 6),
                     "frac_bracketed": round(head["kernel_gbs"] / HBM_PEAK_GBS, 4)},
        "cpu_baseline": cpu,
        "build_info": pa.build_info(),
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
