"""C-ABI library: loads, exports what include/pa.h declares, rejects bad
arguments on the host before touching a device (CPU only, no kernel runs)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pa.h")

pa = pytest.importorskip("prefill_block_table_amd")

P = ctypes.c_void_p
FAKE = ctypes.c_void_p(0x10000)       # aligned, never dereferenced: every call below fails validation
FAKE_MIS = ctypes.c_void_p(0x10002)   # misaligned


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(pa_[a-z_0-9]+)\s*\(", text)))


def _codes():
    text = open(HEADER).read()
    return {m[0]: int(m[1]) for m in re.findall(r"#define (PA_[A-Z_]+) (-?\d+)", text)}


def test_exports_every_declared_symbol():
    names = _declared()
    assert set(names) == {"pa_slot_mapping", "pa_kv_write", "pa_kv_write_fused",
                          "pa_decode_workspace_size", "pa_decode", "pa_decode_append",
                          "pa_prefill_chunk", "pa_prefill_workspace_size", "pa_prefill_varlen",
                          "pa_page_size_for_hybrid", "pa_decode_input_prep",
                          "pa_gemv_bf16", "pa_strerror", "pa_build_info", "pa_decode_noalloc"}
    out = subprocess.run(["nm", "-D", "--defined-only", pa.LIB_PATH], capture_output=True,
                         text=True).stdout
    exported = set(re.findall(r" T (pa_\w+)", out))
    assert set(names) <= exported
    for n in names:
        assert hasattr(pa.lib, n)


def test_build_info_and_strerror():
    info = pa.build_info()
    assert "gfx950" in info and "decode-" in info and "prefill-" in info and "gemv-" in info
    for name, code in _codes().items():
        s = pa.strerror(code)
        assert s and s != "unknown error code", name
    assert pa.strerror(12345) == "unknown error code"


C = _codes()


def _decode(**kw):
    args = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, page_stride=832 * 1024, bt=FAKE, bt_stride=10,
                seq_lens=FAKE, num_seqs=1, max_seq_len=8193, B=832, scale=0.0625, hq=24, hkv=4,
                d=256, ws=FAKE, ws_bytes=1 << 30)
    args.update(kw)
    return pa.lib.pa_decode(args["out"], args["q"], args["k"], args["v"], args["page_stride"],
                            args["bt"], args["bt_stride"], args["seq_lens"], args["num_seqs"],
                            args["max_seq_len"], args["B"], args["scale"], args["hq"],
                            args["hkv"], args["d"], args["ws"], args["ws_bytes"], None)


def test_decode_validation():
    assert _decode(out=None) == C["PA_ERR_NULL"]
    assert _decode(seq_lens=None) == C["PA_ERR_NULL"]
    assert _decode(B=0) == C["PA_ERR_BLOCK_SIZE"]
    assert _decode(d=128) == C["PA_ERR_UNSUPPORTED"]
    assert _decode(hq=32) == C["PA_ERR_UNSUPPORTED"]
    assert _decode(hkv=0, hq=0) == C["PA_ERR_UNSUPPORTED"]
    assert _decode(num_seqs=0) == C["PA_ERR_SIZE"]
    assert _decode(max_seq_len=0) == C["PA_ERR_SIZE"]
    assert _decode(bt_stride=9) == C["PA_ERR_TABLE"]           # 9 * 832 < 8193
    assert _decode(page_stride=832 * 1024 - 8) == C["PA_ERR_STRIDE"]
    assert _decode(q=FAKE_MIS) == C["PA_ERR_ALIGN"]
    assert _decode(k=FAKE_MIS) == C["PA_ERR_ALIGN"]
    assert _decode(ws=None) == C["PA_ERR_WORKSPACE"]
    assert _decode(scale=0.0) == C["PA_ERR_SCALE"]
    assert _decode(scale=-0.0625) == C["PA_ERR_SCALE"]
    assert _decode(scale=float("inf")) == C["PA_ERR_SCALE"]
    assert _decode(scale=float("nan")) == C["PA_ERR_SCALE"]
    need = pa.decode_workspace_size(1, 8193, 832, 4)
    assert _decode(ws_bytes=need - 1) == C["PA_ERR_WORKSPACE"]


def _append(**kw):
    args = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, page_stride=832 * 1024, bt=FAKE, bt_stride=10,
                seq_lens=FAKE, num_seqs=1, max_seq_len=8193, B=832, scale=0.0625, hq=24, hkv=4,
                d=256, k_new=FAKE, v_new=FAKE, slot_out=None, ws=FAKE, ws_bytes=1 << 30)
    args.update(kw)
    return pa.lib.pa_decode_append(args["out"], args["q"], args["k"], args["v"],
                                   args["page_stride"], args["bt"], args["bt_stride"],
                                   args["seq_lens"], args["num_seqs"], args["max_seq_len"],
                                   args["B"], args["scale"], args["hq"], args["hkv"], args["d"],
                                   args["k_new"], args["v_new"], args["slot_out"], args["ws"],
                                   args["ws_bytes"], None)


def test_decode_append_validation():
    assert _append(k_new=None) == C["PA_ERR_NULL"]
    assert _append(v_new=None) == C["PA_ERR_NULL"]
    assert _append(v_new=FAKE_MIS) == C["PA_ERR_ALIGN"]
    assert _append(out=None) == C["PA_ERR_NULL"]
    assert _append(d=128) == C["PA_ERR_UNSUPPORTED"]
    assert _append(bt_stride=9) == C["PA_ERR_TABLE"]
    assert _append(ws=None) == C["PA_ERR_WORKSPACE"]
    assert _append(scale=-1.0) == C["PA_ERR_SCALE"]
    need = pa.decode_workspace_size(1, 8193, 832, 4)
    assert _append(ws_bytes=need - 1) == C["PA_ERR_WORKSPACE"]


def test_workspace_size_monotone():
    a = pa.decode_workspace_size(1, 8193, 832)
    b = pa.decode_workspace_size(16, 32769, 832)
    assert 0 < a < b
    with pytest.raises(pa.PAError):
        pa.decode_workspace_size(0, 10, 16)
    with pytest.raises(pa.PAError):
        pa.decode_workspace_size(1, 10, 0)


def _prefill(**kw):
    args = dict(out=FAKE, q=FAKE, q_len=4096, start=4096, causal=1, k=FAKE, v=FAKE,
                page_stride=832 * 1024, bt=FAKE, n_bt=10, B=832, scale=0.0625, hq=24, hkv=4,
                d=256, ws=None, ws_bytes=0)
    args.update(kw)
    return pa.lib.pa_prefill_chunk(args["out"], args["q"], args["q_len"], args["start"],
                                   args["causal"], args["k"], args["v"], args["page_stride"],
                                   args["bt"], args["n_bt"], args["B"], args["scale"],
                                   args["hq"], args["hkv"], args["d"], args["ws"], args["ws_bytes"],
                                   None)


def test_prefill_validation():
    assert _prefill(q=None) == C["PA_ERR_NULL"]
    assert _prefill(bt=None) == C["PA_ERR_NULL"]
    assert _prefill(B=-1) == C["PA_ERR_BLOCK_SIZE"]
    assert _prefill(d=64) == C["PA_ERR_UNSUPPORTED"]
    assert _prefill(q_len=0) == C["PA_ERR_SIZE"]
    assert _prefill(start=-1) == C["PA_ERR_SIZE"]
    assert _prefill(start=2 ** 31 - 100) == C["PA_ERR_SIZE"]
    assert _prefill(n_bt=9) == C["PA_ERR_TABLE"]               # 9 * 832 < 8192
    assert _prefill(page_stride=100) == C["PA_ERR_STRIDE"]
    assert _prefill(out=FAKE_MIS) == C["PA_ERR_ALIGN"]
    # q=1685 at 8192 splits its last round: a workspace is needed
    need = pa.prefill_workspace_size(1685, 8192, 832)
    assert need > 0 and pa.prefill_workspace_size(4096, 4096, 832) == 0
    assert _prefill(q_len=1685, start=8192, n_bt=12) == C["PA_ERR_WORKSPACE"]
    assert _prefill(q_len=1685, start=8192, n_bt=12, ws=FAKE, ws_bytes=need - 1) == C["PA_ERR_WORKSPACE"]
    assert _prefill(q_len=1685, start=8192, n_bt=12, ws=FAKE_MIS, ws_bytes=need) == C["PA_ERR_ALIGN"]
    assert _prefill(scale=0.0) == C["PA_ERR_SCALE"]
    assert _prefill(scale=-0.0625) == C["PA_ERR_SCALE"]
    assert _prefill(scale=float("nan")) == C["PA_ERR_SCALE"]


def test_kv_write_and_slot_mapping_validation():
    L = pa.lib
    assert L.pa_kv_write(FAKE, FAKE, 832 * 1024, 64, 832, 4, 256, FAKE, FAKE, 1, None, None) == C["PA_ERR_NULL"]
    assert L.pa_kv_write(FAKE, FAKE, 832 * 1024, 64, 832, 4, 128, FAKE, FAKE, 1, FAKE, None) == C["PA_ERR_UNSUPPORTED"]
    assert L.pa_kv_write(FAKE, FAKE, 832 * 1024, 0, 832, 4, 256, FAKE, FAKE, 1, FAKE, None) == C["PA_ERR_SIZE"]
    assert L.pa_kv_write(FAKE, FAKE, 832 * 1024, 64, 832, 4, 256, FAKE, FAKE, -1, FAKE, None) == C["PA_ERR_SIZE"]
    assert L.pa_kv_write(FAKE, FAKE, 832 * 1024, 64, 0, 4, 256, FAKE, FAKE, 1, FAKE, None) == C["PA_ERR_BLOCK_SIZE"]
    assert L.pa_kv_write(FAKE, FAKE, 1024, 64, 832, 4, 256, FAKE, FAKE, 1, FAKE, None) == C["PA_ERR_STRIDE"]
    assert L.pa_kv_write(FAKE, FAKE, 832 * 1024, 64, 832, 4, 256, FAKE_MIS, FAKE, 1, FAKE, None) == C["PA_ERR_ALIGN"]
    # zero tokens: valid, nothing enqueued
    assert L.pa_kv_write(FAKE, FAKE, 832 * 1024, 64, 832, 4, 256, FAKE, FAKE, 0, FAKE, None) == 0
    assert L.pa_kv_write_fused(FAKE, FAKE, 832 * 1024, 64, 832, 4, 256, FAKE, FAKE, 1, None, None, FAKE, 10, None, None) == C["PA_ERR_NULL"]
    assert L.pa_kv_write_fused(FAKE, FAKE, 832 * 1024, 64, 832, 4, 256, FAKE, FAKE, 1, FAKE, None, FAKE, 0, None, None) == C["PA_ERR_SIZE"]
    assert L.pa_kv_write_fused(FAKE, FAKE, 832 * 1024, 64, 832, 4, 256, FAKE, FAKE, 0, FAKE, None, FAKE, 10, None, None) == 0
    assert L.pa_slot_mapping(None, FAKE, None, 1, FAKE, 10, 832, None) == C["PA_ERR_NULL"]
    assert L.pa_slot_mapping(FAKE, FAKE, None, 1, FAKE, 10, 0, None) == C["PA_ERR_BLOCK_SIZE"]
    assert L.pa_slot_mapping(FAKE, FAKE, None, -5, FAKE, 10, 832, None) == C["PA_ERR_SIZE"]
    assert L.pa_slot_mapping(FAKE, FAKE, None, 0, FAKE, 10, 832, None) == 0


def test_decode_input_prep_validation():
    L = pa.lib
    def call(**kw):
        a = dict(sampled=FAKE, pos=100, ids=FAKE, positions=FAKE, mrope=0, stride=0, delta=0,
                 qsl=FAKE, qsl_len=17, sl=FAKE, sl_len=16, mask=FAKE, mask_len=16, itk=None,
                 G=2, bs=FAKE, btp=FAKE, smp=FAKE)
        a.update(kw)
        return L.pa_decode_input_prep(a["sampled"], a["pos"], a["ids"], a["positions"], a["mrope"],
                                      a["stride"], a["delta"], a["qsl"], a["qsl_len"], a["sl"],
                                      a["sl_len"], a["mask"], a["mask_len"], a["itk"], a["G"],
                                      a["bs"], a["btp"], a["smp"], None)
    assert call(sampled=None) == C["PA_ERR_NULL"]
    assert call(ids=None) == C["PA_ERR_NULL"]
    assert call(mask=None) == C["PA_ERR_NULL"]
    assert call(btp=None) == C["PA_ERR_NULL"]
    assert call(pos=-1) == C["PA_ERR_SIZE"]
    assert call(pos=2**31 - 1) == C["PA_ERR_SIZE"]
    assert call(qsl_len=1) == C["PA_ERR_SIZE"]
    assert call(sl_len=0) == C["PA_ERR_SIZE"]
    assert call(G=-1) == C["PA_ERR_SIZE"]
    assert call(mrope=1, stride=0) == C["PA_ERR_SIZE"]


def test_prefill_varlen_validation():
    L = pa.lib
    def call(**kw):
        a = dict(out=FAKE, q=FAKE, total=100, cu=FAKE, su=FAKE, S=3, mq=60, mk=5000, causal=1,
                 k=FAKE, v=FAKE, ps=832 * 1024, bt=FAKE, bts=7, B=832, scale=0.0625, hq=24, hkv=4, d=256)
        a.update(kw)
        return L.pa_prefill_varlen(a["out"], a["q"], a["total"], a["cu"], a["su"], a["S"], a["mq"], a["mk"],
                                   a["causal"], a["k"], a["v"], a["ps"], a["bt"], a["bts"], a["B"],
                                   a["scale"], a["hq"], a["hkv"], a["d"], None)
    assert call(cu=None) == C["PA_ERR_NULL"]
    assert call(su=None) == C["PA_ERR_NULL"]
    assert call(S=0) == C["PA_ERR_SIZE"]
    assert call(mq=0) == C["PA_ERR_SIZE"]
    assert call(total=0) == C["PA_ERR_SIZE"]
    assert call(bts=6) == C["PA_ERR_TABLE"]          # 6 * 832 < 5000
    assert call(scale=-1.0) == C["PA_ERR_SCALE"]
    assert call(hq=32) == C["PA_ERR_UNSUPPORTED"]
    assert call(q=FAKE_MIS) == C["PA_ERR_ALIGN"]
    # (total_q / 128 + num_seqs) * num_q_heads workgroups above 2^31 - 1
    assert call(total=2**31 - 1, hq=384, hkv=64, ps=832 * 64 * 256) == C["PA_ERR_SIZE"]


def test_gemv_validation():
    def call(**kw):
        a = dict(y=FAKE, f32=0, W=FAKE, x=FAKE, N=14336, K=5120, ldw=5120)
        a.update(kw)
        return pa.lib.pa_gemv_bf16(a["y"], a["f32"], a["W"], a["x"], a["N"], a["K"], a["ldw"], None)
    assert call(y=None) == C["PA_ERR_NULL"]
    assert call(W=None) == C["PA_ERR_NULL"]
    assert call(x=None) == C["PA_ERR_NULL"]
    assert call(N=-1) == C["PA_ERR_SIZE"]
    assert call(K=-8) == C["PA_ERR_SIZE"]
    assert call(K=5124, ldw=5128) == C["PA_ERR_SIZE"]
    assert call(ldw=5112) == C["PA_ERR_SIZE"]
    assert call(ldw=5124) == C["PA_ERR_SIZE"]
    assert call(W=FAKE_MIS) == C["PA_ERR_ALIGN"]
    assert call(x=FAKE_MIS) == C["PA_ERR_ALIGN"]
    assert call(y=ctypes.c_void_p(0x10001)) == C["PA_ERR_ALIGN"]
    assert call(y=FAKE_MIS, f32=1) == C["PA_ERR_ALIGN"]
    assert call(N=0, y=None, W=None, x=None) == C["PA_OK"]   # nothing to do, nothing launched


def test_pages_of_4gib_rejected():
    """Rows inside a page are addressed with 32-bit byte offsets: a page of
    one cache of 2^32 bytes or more (block_size * num_kv_heads * 512) is
    rejected before anything is enqueued, by every call that takes a cache."""
    big4 = 2 ** 21                       # 4 KV heads: 2^21 * 4 * 512 = 2^32 bytes
    big64 = 2 ** 17                      # 64 KV heads: 2^17 * 64 * 512 = 2^32 bytes
    assert _decode(B=big4, page_stride=big4 * 1024, bt_stride=1, max_seq_len=100) == C["PA_ERR_BLOCK_SIZE"]
    assert _decode(B=big64, page_stride=big64 * 64 * 256, bt_stride=1, max_seq_len=100, hkv=64,
                   hq=384) == C["PA_ERR_BLOCK_SIZE"]
    assert _append(B=big4, page_stride=big4 * 1024, bt_stride=1, max_seq_len=100) == C["PA_ERR_BLOCK_SIZE"]
    assert _prefill(B=big4, page_stride=big4 * 1024, n_bt=1) == C["PA_ERR_BLOCK_SIZE"]
    assert pa.lib.pa_kv_write(FAKE, FAKE, big4 * 1024, 4, big4, 4, 256, FAKE, FAKE, 1, FAKE,
                              None) == C["PA_ERR_BLOCK_SIZE"]
    # one below the limit passes the page-size check (and fails on a later one)
    assert _decode(B=big4 - 1, page_stride=big4 * 1024, bt_stride=1, max_seq_len=100,
                   ws=None) == C["PA_ERR_WORKSPACE"]


def test_decode_noalloc_rejects_batches_beyond_its_scratch():
    """The allocation-free decode checks the batch against its static 16 MiB
    buffer on the host, before any device call, and validates arguments as
    pa_decode does (its workspace argument aside)."""
    def call(**kw):
        a = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, ps=64 * 1024, bt=FAKE, bts=16, sl=FAKE, S=4000,
                 L=1000, B=64, scale=0.0625, hq=24, hkv=4, d=256)
        a.update(kw)
        return pa.lib.pa_decode_noalloc(a["out"], a["q"], a["k"], a["v"], a["ps"], a["bt"], a["bts"],
                                        a["sl"], a["S"], a["L"], a["B"], a["scale"], a["hq"], a["hkv"],
                                        a["d"], None)
    assert pa.decode_workspace_size(4000, 1000, 64, 4) > (16 << 20)
    assert call() == C["PA_ERR_SCRATCH"]
    assert "scratch" in pa.strerror(C["PA_ERR_SCRATCH"])
    assert call(S=1, out=None) == C["PA_ERR_NULL"]
    assert call(S=1, d=128) == C["PA_ERR_UNSUPPORTED"]
    assert call(S=1, bts=15) == C["PA_ERR_TABLE"]           # 15 * 64 < 1000
    assert call(S=1, scale=-1.0) == C["PA_ERR_SCALE"]
