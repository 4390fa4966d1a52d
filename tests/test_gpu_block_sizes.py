"""GPU parity across block sizes B = 1, 8, 16, 32, 64 (the block-size
trade-off of the pages: "PagedAttention 笔记", block-size discussion, and the
deep-dive page's block-size notes): decode and multi-token attention, bf16,
fp32 and (B >= 16) FP8 pools, against the oracle.  Blocks of fewer than 16
tokens are read in 16-token units made of several blocks; B = 64 in 32-token
units.  Also: a block ID outside the pool skips that block's tokens, for
every block size.
"""
import numpy as np
import pytest

import oracle
import pkv_inputs as pi
from test_gpu_fp8 import check_step, run_fp8
from test_gpu_multi_token import MRun, full_check
from test_gpu_parity import Run, announce, check_attention, dev, host_bits, host_f64, pkv, same_bytes

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pkv().library()
    torch.cuda.set_device(0)


@pytest.mark.parametrize("B", [1, 8, 64])
@pytest.mark.parametrize("dtype,hs,Hq,Hkv", [("bf16", 128, 32, 8), ("bf16", 64, 8, 8), ("f32", 128, 8, 2),
                                             ("f32", 64, 4, 4)])
def test_decode_parity(B, dtype, hs, Hq, Hkv):
    w = pi.make_workload(3, S=7, len_lo=1, len_hi=1400, dtype=dtype, hs=hs, Hq=Hq, Hkv=Hkv, B=B, seed=21)
    announce(f"decode B={B} {dtype} hs={hs} Hq={Hq} Hkv={Hkv} lens={list(w.seq_lens)}")
    r = Run(w)
    slots, kp, vp, ref = oracle.decode_step(w)
    assert np.array_equal(r.slots.cpu().numpy(), slots)
    assert same_bytes(host_bits(r.kc), kp)
    assert same_bytes(host_bits(r.vc), vp)
    check_attention(w, host_f64(r.out), ref)


@pytest.mark.parametrize("B,P", [(1, 16), (1, 48), (1, 80), (1, 208), (1, 512), (8, 16), (8, 128), (64, 64),
                                 (64, 1024)])
def test_partition_lengths(B, P):
    w = pi.make_workload(3, S=5, len_lo=100, len_hi=2000, B=B, seed=22)
    announce(f"decode B={B} P={P} lens={list(w.seq_lens)}")
    r = Run(w, partition_tokens=P)
    check_attention(w, host_f64(r.out), oracle.decode_step(w)[3])


@pytest.mark.parametrize("B", [1, 8, 64])
def test_multi_token_parity(B):
    w0 = pi.make_workload(3, S=6, len_lo=20, len_hi=1200, B=B, seed=23)
    q_lens = np.minimum([1, 4, 17, 40, 3, 64], w0.seq_lens)
    w = pi.make_workload(3, S=6, len_lo=20, len_hi=1200, B=B, seed=23, q_lens=q_lens)
    announce(f"multi-token B={B} lens={list(w.seq_lens)} q_start={list(w.q_start)}")
    full_check(w, MRun(w))


# Lengths at unit and block edges.  With the library's partition length the
# kernel deals a chunk's units (32 tokens for bf16 and FP8 at B = 64, 16 for
# fp32 at B = 32 and 64) to its four waves, so a short sequence can leave a
# wave nothing but units past the sequence's end, or nothing at all.
EDGE_LENS = [1, 16, 17, 31, 32, 33, 48, 63, 64, 65, 96, 97, 128, 129, 160, 191, 192, 193, 255, 256, 257,
             300, 511, 512, 513, 2047, 2049]


@pytest.mark.parametrize("B,dtype,hs", [(64, "bf16", 128), (64, "bf16", 64), (64, "fp8", 128), (32, "f32", 128),
                                        (64, "f32", 128), (64, "f32", 64)])
def test_units_dealt_at_edge_lengths(B, dtype, hs):
    w = pi.make_workload(3, seq_lens=EDGE_LENS, dtype=dtype, B=B, hs=hs, seed=25)
    announce(f"decode B={B} {dtype} hs={hs} edge lengths {list(w.seq_lens)}")
    if dtype == "fp8":
        check_step(w, *run_fp8(w))
        return
    r = Run(w)
    check_attention(w, host_f64(r.out), oracle.decode_step(w)[3])


@pytest.mark.parametrize("B,dtype", [(64, "bf16"), (64, "fp8")])
def test_units_dealt_at_edge_lengths_multi_token(B, dtype):
    q_lens = [min(n, k) for n, k in zip(EDGE_LENS, [1, 2, 5, 16, 33, 3, 64] * 4)]
    w = pi.make_workload(3, seq_lens=EDGE_LENS, dtype=dtype, B=B, seed=26, q_lens=q_lens)
    announce(f"multi-token B={B} {dtype} edge lengths {list(w.seq_lens)} q_start={list(w.q_start)}")
    full_check(w, MRun(w))


@pytest.mark.parametrize("mq", [False, True])
def test_fp8_pools_with_64_token_blocks(mq):
    kw = dict(S=6, len_lo=30, len_hi=1500, B=64, dtype="fp8", seed=24)
    if mq:
        kw["q_lens"] = [2, 5, 1, 9, 16, 3]
    w = pi.make_workload(3, **kw)
    announce(f"fp8 B=64 {'multi-token' if mq else 'decode'} lens={list(w.seq_lens)}")
    if mq:
        full_check(w, MRun(w))
    else:
        check_step(w, *run_fp8(w))
        check_step(w, *run_fp8(w, step=True))


@pytest.mark.parametrize("multi", [False, True])
def test_one_token_blocks_in_windows(multi):
    # B = 1 with 512-token partitions: each wave's block IDs sit in windows of
    # 64; IDs outside the pool at window edges (entries 63, 64, 127 of the
    # first partition, 200, 511) and at the next partition's first entry
    # (512) skip exactly those tokens
    lens = [1100, 700, 90]
    kw = dict(seq_lens=lens, B=1, seed=28)
    if multi:
        kw["q_lens"] = [5, 3, 1]
    w = pi.make_workload(3, **kw)
    bad_at = [63, 64, 127, 200, 511, 512]
    announce(f"B=1 windows: lengths {lens}, out-of-pool IDs at {bad_at}{' (multi-token)' if multi else ''}")
    r = MRun(w) if multi else Run(w)
    m = pkv()
    bt = r.bt.clone()
    for j in bad_at:
        bt[0, j] = -1 - j
    if multi:
        out = m.paged_multi_token_attention(r.q, r.qs, w.max_q_len, r.kc, r.vc, bt, r.sl, w.scale)
    else:
        out = m.paged_decode_attention(r.q, r.kc, r.vc, bt, r.sl, w.scale)
    torch.cuda.synchronize()
    assert m.decode_partition_tokens(w.S, w.Hq, w.Hkv, w.hs, w.M, 1, 0) == 512
    kp, vp = host_bits(r.kc), host_bits(r.vc)
    keep = [j for j in range(w.M) if j not in bad_at]
    tables = np.full_like(w.block_tables, w.block_tables[0, -1])
    tables[0, :len(keep)] = w.block_tables[0, keep]
    tables[1:] = w.block_tables[1:]
    lens2 = w.seq_lens.copy()
    lens2[0] -= len(bad_at)
    if multi:
        # every hole lies below the rows, so on the compacted table each row
        # attends the same tokens as on the original one
        assert max(bad_at) < w.seq_lens[0] - 5
        ref = oracle.paged_multi_token_attention(w.q, w.q_start, kp, vp, tables, lens2, w.scale)
    else:
        ref = oracle.paged_attention(w.q, kp, vp, tables, lens2, w.scale)
    check_attention(w, host_f64(out), ref)


def test_fp8_pools_refuse_small_blocks():
    w = pi.make_workload(3, S=2, len_lo=20, len_hi=40, B=16, dtype="fp8", seed=25)
    m = pkv()
    kc = torch.zeros((4, w.Hkv, w.hs // 16, 8, 16), dtype=torch.uint8, device="cuda")
    vc = torch.zeros((4, w.Hkv, w.hs, 8), dtype=torch.uint8, device="cuda")
    with pytest.raises(m.PkvError):
        m.paged_decode_attention(dev(w.q), kc, vc, dev(w.block_tables), dev(w.seq_lens), w.scale,
                                 k_scale=w.k_scale, v_scale=w.v_scale)


@pytest.mark.parametrize("B", [1, 8, 16, 32, 64])
@pytest.mark.parametrize("bad", [-1, 1 << 30])
def test_block_id_outside_the_pool_skips_its_tokens(B, bad):
    # one full block in the middle of sequence 0 gets an ID outside the pool:
    # the result is attention over the other tokens, i.e. the oracle on the
    # table without that entry and the length shortened by B
    w = pi.make_workload(2, seq_lens=[40 * 8 + 5, 300, 64], B=B, seed=26)
    j = (w.seq_lens[0] // B) // 2
    assert (j + 1) * B <= w.seq_lens[0] - 1  # a full block, not the appended token's
    announce(f"B={B}: block {j} of sequence 0 -> {bad}")
    r = Run(w)
    m = pkv()
    bt = r.bt.clone()
    bt[0, j] = bad
    out = m.paged_decode_attention(r.q, r.kc, r.vc, bt, r.sl, w.scale)
    torch.cuda.synchronize()
    kp, vp = host_bits(r.kc), host_bits(r.vc)
    tables = w.block_tables.copy()
    tables[0, j:-1] = w.block_tables[0, j + 1:]
    lens = w.seq_lens.copy()
    lens[0] -= B
    ref = oracle.paged_attention(w.q, kp, vp, tables, lens, w.scale)
    check_attention(w, host_f64(out), ref)


# The decode step of up to 64 sequences is one launch: the attention takes
# each new token from the step's input while work-groups of the same launch
# store it.  Its output, pools and slots must be those of the separate
# slot-mapping, append and attention calls, bit for bit, in every unit
# shape (16-token tiles, 32-token units, FP8 codes, blocks under 16 tokens)
# and wherever the new token falls in its unit.  Planted: a sequence whose
# last block ID is negative and one whose last block is past the pool (the
# token is neither stored nor attended), and a length past the table row
# (the step attends the row's tokens and stores nothing).
ONE_LAUNCH_CASES = [(1, "bf16", 128), (1, "f32", 64), (8, "bf16", 128), (8, "f32", 128), (8, "bf16", 64),
                    (16, "bf16", 128), (16, "bf16", 64), (16, "f32", 128), (16, "fp8", 128), (16, "fp8", 64),
                    (32, "bf16", 128), (32, "f32", 64), (32, "fp8", 128), (64, "bf16", 128), (64, "bf16", 64),
                    (64, "f32", 128), (64, "fp8", 128), (64, "fp8", 64)]


@pytest.mark.parametrize("P", [None, 64])
@pytest.mark.parametrize("B,dtype,hs", ONE_LAUNCH_CASES)
def test_one_launch_step_bit_identical_to_separate_calls(B, dtype, hs, P):
    lens = EDGE_LENS + [0, 5, 700, 40]
    w = pi.make_workload(3, seq_lens=lens, dtype=dtype, B=B, hs=hs, Hq=8, Hkv=2, seed=27)
    assert w.S <= 64
    bt = w.block_tables.copy()
    sl = w.seq_lens.copy()
    nb = w.k_cache.shape[0]
    bt[28, 4 // B] = -1                     # length 5: last block ID negative
    bt[29, 699 // B] = nb + 3               # length 700: last block past the pool
    sl[30] = w.M * B + 9                    # length past the table row
    part = w.partition_tokens if P is None else P
    announce(f"one-launch decode step B={B} {dtype} hs={hs} P={part} lens={list(sl)}")
    m = pkv()
    sc = dict(k_scale=w.k_scale, v_scale=w.v_scale)
    q, nk, nv, bt_d, sl_d = dev(w.q), dev(w.new_k), dev(w.new_v), dev(bt), dev(sl)
    kc, vc = dev(w.k_cache), dev(w.v_cache)
    slots = torch.full((w.S,), -7, dtype=torch.int64, device="cuda")
    out = m.paged_decode_step(q, nk, nv, kc, vc, bt_d, sl_d, w.scale, slot_mapping=slots, partition_tokens=part, **sc)
    kc2, vc2 = dev(w.k_cache), dev(w.v_cache)
    slots2 = m.decode_slot_mapping(bt_d, sl_d, B)
    m.kv_cache_append(nk, nv, slots2, kc2, vc2, **sc)
    out2 = m.paged_decode_attention(q, kc2, vc2, bt_d, sl_d, w.scale, partition_tokens=part, **sc)
    torch.cuda.synchronize()
    assert torch.equal(slots, slots2)
    assert list(slots2[28:31].cpu().numpy()) == [-1, (nb + 3) * B + 699 % B, -1]
    assert same_bytes(host_bits(kc), host_bits(kc2))
    assert same_bytes(host_bits(vc), host_bits(vc2))
    bits = torch.int16 if out.dtype == torch.bfloat16 else torch.int32
    assert torch.equal(out.view(bits), out2.view(bits))
