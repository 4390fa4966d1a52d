"""Pools of more than 2^31 elements: the blocks a batch uses sit past the
first 2^31 elements of each pool (a 32-bit element offset would wrap), and
the decode step (slot mapping, append, attention with the chunk merge) and
the multi-token step must still read and write exactly them.  The GPU pools
are ~4.3 GiB each; the small workload's blocks are copied to block IDs above
the 2^31-element mark and the tables relabelled, so the oracle runs on the
small pools with the original tables."""
import numpy as np
import pytest

import oracle
import pkv_inputs as pi
from test_gpu_parity import announce, check_attention, dev, host_bits, host_f64, pkv, same_bytes

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pkv().library()
    torch.cuda.set_device(0)


def big_pools(w, shift):
    """GPU pools of w.num_blocks + shift blocks holding w's blocks at id + shift
    (the blocks below are never read: filled with NaN bits once, cheaply)."""
    k_small, v_small = dev(w.k_cache), dev(w.v_cache)
    shape_k = (w.num_blocks + shift,) + tuple(k_small.shape[1:])
    shape_v = (w.num_blocks + shift,) + tuple(v_small.shape[1:])
    fill = 0x7F if k_small.dtype == torch.uint8 else float("nan")  # E4M3 NaN code for FP8 pools
    kc = torch.full(shape_k, fill, dtype=k_small.dtype, device="cuda")
    vc = torch.full(shape_v, fill, dtype=v_small.dtype, device="cuda")
    kc[shift:].copy_(k_small)
    vc[shift:].copy_(v_small)
    return kc, vc


@pytest.mark.parametrize("cfg,kw", [(3, dict(S=6, len_lo=600, len_hi=3000)), (4, dict(S=1, len_lo=5000, len_hi=9000)),
                                    (3, dict(S=5, len_lo=600, len_hi=3000, dtype="fp8"))])
def test_decode_step_past_2g_elements(cfg, kw):
    w = pi.make_workload(cfg, **kw)
    per_block = w.Hkv * w.hs * w.B
    shift = (1 << 31) // per_block + 7  # first used block starts past element 2^31
    announce(f"pools of {(w.num_blocks + shift) * per_block} elements: config {cfg} lens={list(w.seq_lens)}")
    m = pkv()
    kc, vc = big_pools(w, shift)
    bt = w.block_tables.astype(np.int64) + shift
    assert bt.max() * per_block >= (1 << 31)
    bt_dev = torch.from_numpy(bt.astype(np.int32)).cuda()
    q, sl, nk, nv = dev(w.q), dev(w.seq_lens), dev(w.new_k), dev(w.new_v)
    slots = torch.empty(w.S, dtype=torch.int64, device="cuda")
    out = m.paged_decode_step(q, nk, nv, kc, vc, bt_dev, sl, w.scale, slot_mapping=slots, k_scale=w.k_scale,
                              v_scale=w.v_scale)
    torch.cuda.synchronize()
    ref_slots, kp, vp, ref = oracle.decode_step(w)
    assert np.array_equal(slots.cpu().numpy(), np.where(ref_slots >= 0, ref_slots + shift * w.B, ref_slots))
    check_attention(w, host_f64(out), ref)
    assert same_bytes(host_bits(kc[shift:]), kp), "key pool differs after the append"
    assert same_bytes(host_bits(vc[shift:]), vp), "value pool differs after the append"


def test_multi_token_step_past_2g_elements():
    w = pi.make_workload(3, S=4, len_lo=300, len_hi=2500, q_lens=[40, 3, 17, 1])
    per_block = w.Hkv * w.hs * w.B
    shift = (1 << 31) // per_block + 3
    announce(f"multi-token step on pools of {(w.num_blocks + shift) * per_block} elements")
    m = pkv()
    kc, vc = big_pools(w, shift)
    bt_dev = torch.from_numpy((w.block_tables.astype(np.int64) + shift).astype(np.int32)).cuda()
    q, sl, qs, nk, nv = dev(w.q), dev(w.seq_lens), dev(w.q_start), dev(w.new_k), dev(w.new_v)
    out = m.paged_multi_token_step(q, nk, nv, kc, vc, qs, w.max_q_len, bt_dev, sl, w.scale)
    torch.cuda.synchronize()
    _, kp, vp, ref = oracle.multi_token_step(w)
    check_attention(w, host_f64(out), ref)
    assert same_bytes(host_bits(kc[shift:]), kp) and same_bytes(host_bits(vc[shift:]), vp)
    # the unpartitioned kernel on the same pools
    out_u = m.paged_multi_token_attention(q, qs, w.max_q_len, kc, vc, bt_dev, sl, w.scale,
                                          partition_tokens=m.PARTITION_NONE)
    torch.cuda.synchronize()
    check_attention(w, host_f64(out_u), ref)


def test_copy_blocks_past_2g_elements():
    # copy-on-write copies between blocks past element 2^31: whole blocks of
    # both pools, the other blocks untouched
    w = pi.make_workload(3, S=2, len_lo=300, len_hi=600)
    per_block = w.Hkv * w.hs * w.B
    shift = (1 << 31) // per_block + 11
    announce(f"block copies on pools of {(w.num_blocks + shift) * per_block} elements")
    m = pkv()
    kc, vc = big_pools(w, shift)
    src = np.array([0, 5, w.num_blocks - 1]) + shift
    dst = np.array([w.num_blocks - 2, 9, 3]) + shift
    before_k, before_v = kc.clone(), vc.clone()
    pairs = torch.from_numpy(np.stack([src, dst], 1).astype(np.int32)).cuda()  # [n, 2]
    m.copy_blocks(pairs, kc, vc)
    torch.cuda.synchronize()
    bits = (lambda t: t.view(torch.int16))
    for a, b in zip(src, dst):
        assert torch.equal(bits(kc[b]), bits(before_k[a])) and torch.equal(bits(vc[b]), bits(before_v[a]))
    untouched = [i for i in range(shift, shift + w.num_blocks) if i not in set(dst.tolist())][:4] + [shift - 1]
    for i in untouched:
        assert torch.equal(bits(kc[i]), bits(before_k[i])) and torch.equal(bits(vc[i]), bits(before_v[i]))
