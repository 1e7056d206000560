"""GPU parity: slot mapping and KV-cache write, bit-exact against the oracle."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import bits, log, to_dev

pytestmark = pytest.mark.gpu


def _pa():
    import prefill_block_table_amd as pa
    return pa


def _sync():
    import torch
    torch.cuda.synchronize()


@pytest.mark.parametrize("B", [1, 16, 784, 832, 1024])
def test_slot_mapping_bit_exact(B):
    pa = _pa()
    rng = np.random.default_rng(B)
    S, maxp = 5, 12
    num_pages = S * maxp + 3
    bt = rng.permutation(num_pages)[: S * maxp].reshape(S, maxp).astype(np.int32)
    T = 777
    seq = rng.integers(0, S, T).astype(np.int32)
    pos = rng.integers(0, maxp * B, T).astype(np.int64)
    pos[:3] = [0, maxp * B - 1, B]
    bad = np.zeros(T, bool)
    pos[3], bad[3] = -1, True             # negative position -> -1
    pos[4], bad[4] = maxp * B, True       # logical page past the table -> -1
    log(f"slot_mapping B={B} T={T}")
    got = pa.slot_mapping(to_dev(pos), to_dev(bt), B, token_seq=to_dev(seq)).cpu().numpy()
    ref = np.full(T, -1, np.int64)
    ref[~bad] = oracle.slot_mapping(pos[~bad], seq[~bad], bt, B)
    assert np.array_equal(got, ref)


def _poison_pool(P, B, H=4, fill=W.BF16_QNAN):
    return (np.full((P, B, H, 256), fill, np.uint16), np.full((P, B, H, 256), fill ^ 0x8000, np.uint16))


def test_kv_write_bit_exact_with_skipped_slots():
    pa = _pa()
    rng = np.random.default_rng(3)
    P, B, T = 9, 100, 300
    k0, v0 = _poison_pool(P, B)
    kn = W.normal_bf16(rng, (T, 4, 256))
    vn = W.normal_bf16(rng, (T, 4, 256))
    slots = rng.permutation(P * B)[:T].astype(np.int64)
    slots[:4] = [-1, P * B, 10 ** 12, 0]
    log("kv_write P=9 B=100 T=300 with invalid slots")
    k, v = to_dev(k0), to_dev(v0)
    pa.kv_write(k, v, to_dev(kn), to_dev(vn), to_dev(slots))
    _sync()
    rk, rv = oracle.kv_write(k0, v0, kn, vn, slots)
    assert np.array_equal(bits(k), rk) and np.array_equal(bits(v), rv)


@pytest.mark.parametrize("hkv", [1, 4, 8])
def test_kv_write_fused_bit_exact(hkv):
    pa = _pa()
    rng = np.random.default_rng(4 + hkv)
    S, B, maxp = 3, 784, 4
    P = S * maxp + 2
    bt = rng.permutation(P)[: S * maxp].reshape(S, maxp).astype(np.int32)
    T = 50
    seq = rng.integers(0, S, T).astype(np.int32)
    pos = rng.permutation(maxp * B)[:T].astype(np.int64)   # distinct positions per sequence
    k0, v0 = _poison_pool(P, B, hkv)
    kn = W.normal_bf16(rng, (T, hkv, 256))
    vn = W.normal_bf16(rng, (T, hkv, 256))
    log(f"kv_write_fused hkv={hkv}")
    k, v = to_dev(k0), to_dev(v0)
    import torch
    slot_out = torch.full((T,), -7, dtype=torch.int64, device=k.device)
    pa.kv_write_fused(k, v, to_dev(kn), to_dev(vn), to_dev(pos), to_dev(bt), to_dev(seq), slot_out)
    _sync()
    slots = oracle.slot_mapping(pos, seq, bt, B)
    rk, rv = oracle.kv_write(k0, v0, kn, vn, slots)
    assert np.array_equal(slot_out.cpu().numpy(), slots)
    assert np.array_equal(bits(k), rk) and np.array_equal(bits(v), rv)


def test_kv_write_joint_page_layout():
    """K and V as views of one [P, 2, B, Hkv, D] tensor (page stride 2 pages)."""
    import torch
    pa = _pa()
    rng = np.random.default_rng(5)
    P, B, T = 6, 64, 40
    joint0 = np.full((P, 2, B, 4, 256), W.BF16_QNAN, np.uint16)
    kn = W.normal_bf16(rng, (T, 4, 256))
    vn = W.normal_bf16(rng, (T, 4, 256))
    slots = rng.permutation(P * B)[:T].astype(np.int64)
    log("kv_write joint layout")
    joint = to_dev(joint0)
    pa.kv_write(joint[:, 0], joint[:, 1], to_dev(kn), to_dev(vn), to_dev(slots))
    torch.cuda.synchronize()
    rk, rv = oracle.kv_write(joint0[:, 0], joint0[:, 1], kn, vn, slots)
    got = bits(joint)
    assert np.array_equal(got[:, 0], rk) and np.array_equal(got[:, 1], rv)


@pytest.mark.parametrize("which", ["decode_8k", "batched_decode", "prefill_chunk_a"])
def test_workload_writes_bit_exact(which):
    pa = _pa()
    if which == "prefill_chunk_a":
        c = W.prefill_8k()
        ch = c.chunks[0]
        bt = c.block_table[None]
        pos = np.arange(ch.start_pos, ch.start_pos + ch.q_len, dtype=np.int64)
        seq = np.zeros(ch.q_len, np.int32)
        kn, vn = ch.k_new, ch.v_new
        k0, v0, B = c.k_cache, c.v_cache, c.block_size
    else:
        c = W.decode_8k() if which == "decode_8k" else W.batched_decode()
        bt, pos, seq, kn, vn = c.block_tables, c.positions, c.token_seq, c.k_new, c.v_new
        k0, v0, B = c.k_cache, c.v_cache, c.block_size
    log(f"workload write {which}: T={len(pos)}")
    k, v = to_dev(k0), to_dev(v0)
    pa.kv_write_fused(k, v, to_dev(kn), to_dev(vn), to_dev(pos), to_dev(bt), to_dev(seq))
    _sync()
    slots = oracle.slot_mapping(pos, seq, bt, B)
    rk, rv = oracle.kv_write(k0, v0, kn, vn, slots)
    assert np.array_equal(bits(k), rk) and np.array_equal(bits(v), rv)
