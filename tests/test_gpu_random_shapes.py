"""Seeded random small shapes through the whole decode step and the whole
multi-token step, against the oracle: element type, head size, block size,
group size, batch size, lengths (with empty sequences, one-token ones and
full tables) and partition length drawn from a fixed seed, so the cases are
the same on every run.  Appends bit-exact, outputs within the bars."""
import os

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


def draw_case(rng, multi, unpartitioned=False):
    dtype = ["f32", "bf16", "bf16", "fp8"][rng.integers(4)]
    if unpartitioned:
        dtype = ["bf16", "fp8"][rng.integers(2)]
    hs = [64, 128][rng.integers(2)]
    blocks = [16, 32, 64] if (dtype == "fp8" or unpartitioned) else [1, 8, 16, 32, 64]
    B = blocks[rng.integers(len(blocks))]
    Hkv = [1, 2, 4, 8][rng.integers(4)]
    G = [1, 2, 4, 8][rng.integers(4)]
    S = int(rng.integers(1, 41))
    cap = 1500 if B == 1 else 2500
    lens = rng.integers(1, cap, S)
    for k in range(S):  # some special lengths
        u = rng.random()
        lens[k] = 0 if u < 0.08 else (1 if u < 0.14 else (B if u < 0.2 else lens[k]))
    if S > 1 and lens.max() == 0:
        lens[0] = 5
    # partition length: the library's, or a requested one that fits the block size
    P = 0
    if rng.random() < 0.4:
        mult = B if B >= 16 else 16
        P = int(mult * rng.integers(1, max(2, (64 * B) // mult + 1)))
        P = min(P, 64 * B)
    q_lens = None
    if multi:
        q_lens = [int(min(L, rng.integers(1, 24))) if L > 0 else 0 for L in lens]
        if unpartitioned:
            P = -1  # the unpartitioned kernel
    return dict(dtype=dtype, hs=hs, B=B, Hkv=Hkv, Hq=Hkv * G, seq_lens=[int(x) for x in lens], q_lens=q_lens, P=P)


def draw_long_rows(rng):
    """A case for the unpartitioned kernel with many rows per sequence."""
    dtype = ["bf16", "fp8"][rng.integers(2)]
    hs = [64, 128][rng.integers(2)]
    B = [16, 32, 64][rng.integers(3)]
    Hkv = [1, 2, 4][rng.integers(3)]
    G = [1, 2, 4][rng.integers(3)]
    lens = rng.integers(64, 2000, int(rng.integers(1, 7)))
    q_lens = [int(min(L, rng.integers(16, 200))) for L in lens]
    return dict(dtype=dtype, hs=hs, B=B, Hkv=Hkv, Hq=Hkv * G, seq_lens=[int(x) for x in lens], q_lens=q_lens, P=-1)


def draw_wide(rng, multi):
    """A case on the paths draw_case leaves rare: half of them batches of
    65-300 sequences (the schedule's chunk list), each through either the
    whole step or the stand-alone attention on the appended pools without a
    schedule, and half of the bf16 / FP8 ones with an fp32 output."""
    c = draw_case(rng, multi)
    if rng.random() < 0.5:
        S = int(rng.integers(65, 301))
        lens = rng.integers(1, 800 if c["B"] == 1 else 2500, S)
        for k in range(S):
            u = rng.random()
            lens[k] = 0 if u < 0.05 else (1 if u < 0.1 else lens[k])
        c["seq_lens"] = [int(x) for x in lens]
        c["Hq"] = c["Hkv"] * min(c["Hq"] // c["Hkv"], 4)
        if multi:
            c["q_lens"] = [int(min(L, rng.integers(1, 12))) if L > 0 else 0 for L in lens]
    c["mode"] = ["step", "attn"][rng.integers(2)]
    c["f32out"] = c["dtype"] != "f32" and bool(rng.random() < 0.5)
    return c


_rng = np.random.default_rng(20260211)
DECODE = [draw_case(_rng, False) for _ in range(24)]
MULTI = [draw_case(_rng, True) for _ in range(12)] + [draw_case(_rng, True, unpartitioned=True) for _ in range(4)]
# More cases on request: PKV_RANDOM_CASES="seed:decode:multi:long" draws that
# many decode-step, multi-token-step and long-row cases from the given seed
# (for example "4242:1500:600:200", a few minutes on one GPU).
_extra = os.environ.get("PKV_RANDOM_CASES")
if _extra:
    _seed, _nd, _nm, _nl = (int(x) for x in _extra.split(":"))
    _erng = np.random.default_rng(_seed)
    DECODE += [draw_case(_erng, False) for _ in range(_nd)]
    MULTI += [draw_case(_erng, True) for _ in range(_nm)] + [draw_long_rows(_erng) for _ in range(_nl)]
# PKV_RANDOM_WIDE="seed:decode:multi": cases from draw_wide (large batches,
# stand-alone attention without a schedule, fp32 outputs)
WIDE = []
_wide = os.environ.get("PKV_RANDOM_WIDE")
if _wide:
    _seed, _nd, _nm = (int(x) for x in _wide.split(":"))
    _wrng = np.random.default_rng(_seed)
    WIDE = [draw_wide(_wrng, False) for _ in range(_nd)] + [draw_wide(_wrng, True) for _ in range(_nm)]


def case_id(c):
    return f"{c['dtype']}-hs{c['hs']}-B{c['B']}-{c['Hq']}x{c['Hkv']}-S{len(c['seq_lens'])}-P{c['P']}"


def workload(c):
    kw = dict(dtype=c["dtype"], hs=c["hs"], B=c["B"], Hq=c["Hq"], Hkv=c["Hkv"], seq_lens=c["seq_lens"])
    if c["q_lens"] is not None:
        kw["q_lens"] = c["q_lens"]
    return pi.make_workload(3, **kw)


@pytest.mark.parametrize("c", DECODE, ids=[case_id(c) for c in DECODE])
def test_random_decode_step(c):
    w = workload(c)
    announce(f"random decode step {case_id(c)} lens={c['seq_lens']}")
    m = pkv()
    q, kc, vc, bt, sl = dev(w.q), dev(w.k_cache), dev(w.v_cache), dev(w.block_tables), dev(w.seq_lens)
    slots = torch.empty(w.S, dtype=torch.int64, device="cuda")
    out = m.paged_decode_step(q, dev(w.new_k), dev(w.new_v), kc, vc, bt, sl, w.scale, slot_mapping=slots,
                              partition_tokens=c["P"], k_scale=w.k_scale, v_scale=w.v_scale)
    torch.cuda.synchronize()
    ref_slots, kp, vp, ref = oracle.decode_step(w)
    assert np.array_equal(slots.cpu().numpy(), ref_slots)
    assert same_bytes(host_bits(kc), kp) and same_bytes(host_bits(vc), vp)
    check_attention(w, host_f64(out), ref)


@pytest.mark.parametrize("c", MULTI, ids=[case_id(c) for c in MULTI])
def test_random_multi_token_step(c):
    w = workload(c)
    announce(f"random multi-token step {case_id(c)} lens={c['seq_lens']} q_lens={c['q_lens']}")
    m = pkv()
    q, kc, vc, bt, sl, qs = (dev(w.q), dev(w.k_cache), dev(w.v_cache), dev(w.block_tables), dev(w.seq_lens),
                             dev(w.q_start))
    slots = torch.empty(w.rows, dtype=torch.int64, device="cuda")
    out = m.paged_multi_token_step(q, dev(w.new_k), dev(w.new_v), kc, vc, qs, w.max_q_len, bt, sl, w.scale,
                                   slot_mapping=slots, partition_tokens=c["P"], k_scale=w.k_scale,
                                   v_scale=w.v_scale)
    torch.cuda.synchronize()
    ref_slots, kp, vp, ref = oracle.multi_token_step(w)
    assert np.array_equal(slots.cpu().numpy(), ref_slots)
    assert same_bytes(host_bits(kc), kp) and same_bytes(host_bits(vc), vp)
    check_attention(w, host_f64(out), ref)


def check_wide(c):
    multi = c["q_lens"] is not None
    w = workload(c)
    announce(f"random {'multi-token' if multi else 'decode'} {c['mode']} {case_id(c)} f32out={c['f32out']}")
    m = pkv()
    sc = dict(k_scale=w.k_scale, v_scale=w.v_scale, partition_tokens=c["P"],
              out_dtype=torch.float32 if c["f32out"] else None)
    ref_slots, kp, vp, ref = oracle.multi_token_step(w) if multi else oracle.decode_step(w)
    bt, sl = dev(w.block_tables), dev(w.seq_lens)
    if c["mode"] == "step":
        kc, vc = dev(w.k_cache), dev(w.v_cache)
        slots = torch.empty(w.rows if multi else w.S, dtype=torch.int64, device="cuda")
        if multi:
            out = m.paged_multi_token_step(dev(w.q), dev(w.new_k), dev(w.new_v), kc, vc, dev(w.q_start), w.max_q_len,
                                           bt, sl, w.scale, slot_mapping=slots, **sc)
        else:
            out = m.paged_decode_step(dev(w.q), dev(w.new_k), dev(w.new_v), kc, vc, bt, sl, w.scale,
                                      slot_mapping=slots, **sc)
        torch.cuda.synchronize()
        assert np.array_equal(slots.cpu().numpy(), ref_slots)
        assert same_bytes(host_bits(kc), kp) and same_bytes(host_bits(vc), vp)
    else:  # the attention alone on the appended pools, no schedule
        if multi:
            out = m.paged_multi_token_attention(dev(w.q), dev(w.q_start), w.max_q_len, dev(kp), dev(vp), bt, sl,
                                                w.scale, **sc)
        else:
            out = m.paged_decode_attention(dev(w.q), dev(kp), dev(vp), bt, sl, w.scale, **sc)
        torch.cuda.synchronize()
    check_attention(w, host_f64(out), ref, out_f32=c["f32out"])


if WIDE:  # defined only on request, so a default run has no empty parameter set
    @pytest.mark.parametrize("c", WIDE, ids=[f"{c['mode']}{'-f32out' if c['f32out'] else ''}-{case_id(c)}"
                                             for c in WIDE])
    def test_random_wide(c):
        check_wide(c)
