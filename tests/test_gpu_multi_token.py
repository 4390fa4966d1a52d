"""GPU parity of attention with several query tokens per sequence (chunked
prefill, prefix-miss prefill, speculative decoding) against the oracle.

Rule: the n_s query rows of sequence s are its last n_s tokens, row i at
position L_s - n_s + i attends the positions up to its own.  The rows' own
keys and values are appended first (slot mapping + append, bit-exact), as in
a decode step.  Bars as for decode: max-abs error <= 1e-5 (fp32) and <= 2e-3
(bf16 outputs, with the half-ulp rule for |out| >= 1), appends bit-exact.
"""
from types import SimpleNamespace

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


class MRun:
    """Slot mapping + append + attention through the separate entry points."""

    def __init__(self, w, partition_tokens=None, max_q_len=None):
        self.w = w
        P = w.partition_tokens if partition_tokens is None else partition_tokens
        self.mql = w.max_q_len if max_q_len is None else max_q_len
        m = pkv()
        self.q, self.kc, self.vc = dev(w.q), dev(w.k_cache), dev(w.v_cache)
        self.bt, self.sl, self.qs = dev(w.block_tables), dev(w.seq_lens), dev(w.q_start)
        self.nk, self.nv = dev(w.new_k), dev(w.new_v)
        self.slots = m.multi_token_slot_mapping(self.bt, self.sl, self.qs, w.rows, self.mql, w.B)
        m.kv_cache_append(self.nk, self.nv, self.slots, self.kc, self.vc, k_scale=w.k_scale, v_scale=w.v_scale)
        self.out = m.paged_multi_token_attention(self.q, self.qs, self.mql, self.kc, self.vc, self.bt, self.sl,
                                                 w.scale, partition_tokens=P, k_scale=w.k_scale, v_scale=w.v_scale)
        torch.cuda.synchronize()


def full_check(w, r):
    slots, kp, vp, ref = oracle.multi_token_step(w)
    assert np.array_equal(r.slots.cpu().numpy(), slots)
    assert same_bytes(host_bits(r.kc), kp), "key pool differs after append"
    assert same_bytes(host_bits(r.vc), vp), "value pool differs after append"
    check_attention(w, host_f64(r.out), ref)


CASES = [
    # (config, overrides): full prefill from position 0, chunks, drafts, single rows
    (1, dict(q_lens=[35, 16, 1, 50])),
    (1, dict(q_lens=[5, 3, 1, 17])),
    (2, dict(S=5, len_lo=100, len_hi=700, q_lens=[8, 1, 33, 2, 16])),
    (3, dict(S=12, len_lo=16, len_hi=1500, q_lens=4)),
    (3, dict(S=6, len_lo=300, len_hi=2500, q_lens=[64, 5, 1, 37, 128, 16])),
    (4, dict(S=2, len_lo=1500, len_hi=5000, q_lens=[7, 24])),
    (5, dict(S=8, len_hi=256, q_lens=3)),
    (3, dict(S=6, len_lo=100, len_hi=1300, dtype="fp8", q_lens=[4, 9, 1, 16, 2, 30])),
    (4, dict(S=2, len_lo=700, len_hi=3000, dtype="fp8", q_lens=[5, 12])),
]


@pytest.mark.parametrize("cfg,kw", CASES)
def test_small_multi_token_parity(cfg, kw):
    w = pi.make_workload(cfg, **kw)
    announce(f"multi-token config {cfg} {w.dtype}: lens={list(w.seq_lens)} q_start={list(w.q_start)} B={w.B} G={w.G}")
    full_check(w, MRun(w))


@pytest.mark.parametrize("P", [16, 64, 128])
def test_partition_lengths_and_chunk_merge(P):
    # short partitions: many chunks per sequence, so the chunk-merge kernel
    # combines per-row partials, some of which see no token of a row
    w = pi.make_workload(3, S=4, len_lo=200, len_hi=900, q_lens=[40, 3, 17, 1])
    announce(f"multi-token partitions of {P}: lens={list(w.seq_lens)}")
    full_check(w, MRun(w, partition_tokens=P))


@pytest.mark.parametrize("dtype,hs,B,Hq,Hkv", [
    ("f32", 64, 16, 8, 8), ("f32", 128, 32, 8, 2), ("bf16", 64, 16, 8, 8), ("bf16", 64, 32, 16, 2),
    ("bf16", 128, 16, 16, 1), ("bf16", 128, 32, 12, 4), ("bf16", 64, 16, 24, 8),
])
def test_shape_sweep(dtype, hs, B, Hq, Hkv):
    w = pi.make_workload(3, S=5, len_lo=1, len_hi=700, dtype=dtype, hs=hs, B=B, Hq=Hq, Hkv=Hkv,
                         seed=11, q_lens=None)
    q_lens = np.minimum(np.array([1, 6, 13, 2, 40]), w.seq_lens)
    w = pi.make_workload(3, S=5, len_lo=1, len_hi=700, dtype=dtype, hs=hs, B=B, Hq=Hq, Hkv=Hkv, seed=11,
                         q_lens=q_lens)
    announce(f"multi-token shapes {dtype} hs={hs} B={B} Hq={Hq} Hkv={Hkv} q_start={list(w.q_start)}")
    full_check(w, MRun(w))


def test_one_row_each_is_bit_identical_to_decode():
    w = pi.make_workload(3, S=12, len_lo=16, len_hi=2500, q_lens=1)
    announce("multi-token with one row per sequence vs decode attention")
    r = MRun(w)
    m = pkv()
    out = m.paged_decode_attention(r.q, r.kc, r.vc, r.bt, r.sl, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), r.out.view(torch.int16))


def test_sequences_without_rows_and_a_larger_max_q_len():
    # sequences with no query rows in the batch, an empty sequence, and
    # max_q_len above every n: rows are exactly those of q_start
    lens = [40, 0, 17, 300, 5]
    q_lens = [3, 0, 0, 21, 5]
    w = pi.make_workload(2, seq_lens=lens, q_lens=q_lens)
    announce(f"rows {q_lens} of lengths {lens}, max_q_len 64")
    r = MRun(w, max_q_len=64)
    full_check(w, r)


@pytest.mark.parametrize("lens", [[0], [0, 12, 300]])
def test_a_batch_without_any_rows_does_nothing(lens):
    # every sequence sits the step out: q, out and the new rows are empty,
    # the pools are left as they are
    w = pi.make_workload(2, seq_lens=lens, q_lens=[0] * len(lens))
    announce(f"no rows at all, lengths {lens}")
    assert w.rows == 0
    m = pkv()
    q, kc, vc, bt, sl, qs = dev(w.q), dev(w.k_cache), dev(w.v_cache), dev(w.block_tables), dev(w.seq_lens), \
        dev(w.q_start)
    kc0, vc0 = kc.clone(), vc.clone()
    for mql in (0, 4):
        out = m.paged_multi_token_step(q, dev(w.new_k), dev(w.new_v), kc, vc, qs, mql, bt, sl, w.scale)
        out2 = m.paged_multi_token_attention(q, qs, mql, kc, vc, bt, sl, w.scale)
        torch.cuda.synchronize()
        assert out.numel() == 0 and out2.numel() == 0
    assert torch.equal(kc.view(torch.uint8), kc0.view(torch.uint8))
    assert torch.equal(vc.view(torch.uint8), vc0.view(torch.uint8))


def test_step_matches_the_separate_calls():
    w = pi.make_workload(3, S=6, len_lo=300, len_hi=2500, q_lens=[64, 5, 1, 37, 128, 16])
    announce("multi-token step vs slot mapping + append + attention")
    r = MRun(w)
    m = pkv()
    kc, vc = dev(w.k_cache), dev(w.v_cache)
    slots = torch.empty(w.rows, dtype=torch.int64, device="cuda")
    out = m.paged_multi_token_step(r.q, r.nk, r.nv, kc, vc, r.qs, w.max_q_len, r.bt, r.sl, w.scale,
                                   slot_mapping=slots)
    torch.cuda.synchronize()
    assert torch.equal(slots, r.slots)
    assert torch.equal(kc.view(torch.int16), r.kc.view(torch.int16))
    assert torch.equal(vc.view(torch.int16), r.vc.view(torch.int16))
    assert torch.equal(out.view(torch.int16), r.out.view(torch.int16))


def sampled_rows_reference(w, kp, vp, picks):
    """Oracle rows for sampled (sequence, row) pairs: row i of sequence s is
    a one-token query at position L - n + i, i.e. decode attention over the
    first L - n + i + 1 tokens of the same table row."""
    q = np.stack([w.q[w.q_start[s] + i] for s, i in picks])
    tables = np.stack([w.block_tables[s] for s, _ in picks])
    lens = np.array([w.seq_lens[s] - (w.q_start[s + 1] - w.q_start[s]) + i + 1 for s, i in picks], np.int32)
    if w.dtype == "fp8":
        return oracle.paged_attention_fp8(q, kp, vp, tables, lens, w.scale, w.k_scale, w.v_scale)
    return oracle.paged_attention(q, kp, vp, tables, lens, w.scale)


@pytest.mark.parametrize("kind", ["spec4", "chunk512"])
def test_full_size_rows(kind):
    # the benchmark's multi-token workloads on the GQA configuration: 4 draft
    # tokens for each of the 256 sequences (every row and query head
    # compared), or the last (up to) 512 tokens of each as a prefill chunk
    # (every row of four whole sequences -- the longest, the shortest and two
    # drawn ones -- and three rows of 24 more: the oracle's plain loops take
    # about 1.5 minutes on 16 threads for all 122k rows)
    base = pi.make_workload(3)
    n = 4 if kind == "spec4" else 512
    w = pi.make_workload(3, q_lens=np.minimum(n, base.seq_lens))
    del base
    announce(f"full-size multi-token {kind}: rows={w.rows} max_q_len={w.max_q_len}")
    r = MRun(w)
    slots = oracle.multi_token_slot_mapping(w.block_tables, w.seq_lens, w.q_start, w.B)
    assert np.array_equal(r.slots.cpu().numpy(), slots)
    kp, vp = w.k_cache.copy(), w.v_cache.copy()
    oracle.kv_append(w.new_k, w.new_v, slots, kp, vp)
    assert same_bytes(host_bits(r.kc), kp)
    assert same_bytes(host_bits(r.vc), vp)
    if kind == "spec4":
        ref = oracle.paged_multi_token_attention(w.q, w.q_start, kp, vp, w.block_tables, w.seq_lens, w.scale)
        check_attention(w, host_f64(r.out), ref)
    else:
        g = np.random.default_rng(5)
        ns = np.diff(w.q_start)
        whole = [int(np.argmax(w.seq_lens)), int(np.argmin(w.seq_lens))]
        whole += [int(s) for s in g.choice(np.setdiff1d(np.arange(w.S), whole), size=2, replace=False)]
        picks = [(s, i) for s in whole for i in range(int(ns[s]))]
        for s in g.choice(np.setdiff1d(np.arange(w.S), whole), size=24, replace=False):
            for i in {0, int(ns[s]) - 1, int(g.integers(0, ns[s]))}:
                picks.append((int(s), i))
        announce(f"  {len(picks)} rows compared ({len(whole)} whole sequences)")
        ref = sampled_rows_reference(w, kp, vp, picks)
        got = host_f64(r.out)[[w.q_start[s] + i for s, i in picks]]
        check_attention(w, got, ref)
    assert torch.isfinite(r.out.float()).all().item()


PREFILL_CASES = [c for c in CASES if c[1].get("dtype", pi._CFG[c[0]]["dtype"]) != "f32"] + [
    # rows spanning several 128-row blocks, long contexts, both block sizes
    (3, dict(S=3, len_lo=600, len_hi=2500, q_lens=[300, 64, 129])),
    (4, dict(S=1, len_lo=3000, len_hi=3000, q_lens=[200])),
    (2, dict(S=2, len_lo=900, len_hi=1200, q_lens=[900, 130])),
    (3, dict(S=3, len_lo=200, len_hi=700, dtype="fp8", q_lens=[100, 37, 150])),
]


@pytest.mark.parametrize("cfg,kw", PREFILL_CASES)
def test_unpartitioned_kernel_parity(cfg, kw):
    w = pi.make_workload(cfg, **kw)
    announce(f"unpartitioned multi-token config {cfg} {w.dtype}: lens={list(w.seq_lens)} q_start={list(w.q_start)} "
             f"B={w.B} G={w.G}")
    full_check(w, MRun(w, partition_tokens=pkv().PARTITION_NONE))


@pytest.mark.parametrize("B", [16, 32, 64])
def test_unpartitioned_kernel_block_sizes_and_a_skipped_block(B):
    w = pi.make_workload(3, S=3, len_lo=300, len_hi=900, B=B, seed=31, q_lens=[40, 100, 7])
    announce(f"unpartitioned B={B}: lens={list(w.seq_lens)}")
    r = MRun(w, partition_tokens=pkv().PARTITION_NONE)
    full_check(w, r)
    # a block ID outside the pool in sequence 1 (a full block before the rows):
    # its tokens are skipped, the same as the oracle on the table without it
    m = pkv()
    j = 1
    bt = r.bt.clone()
    bt[1, j] = -3
    out = m.paged_multi_token_attention(r.q, r.qs, w.max_q_len, r.kc, r.vc, bt, r.sl, w.scale,
                                        partition_tokens=m.PARTITION_NONE)
    out_p = m.paged_multi_token_attention(r.q, r.qs, w.max_q_len, r.kc, r.vc, bt, r.sl, w.scale,
                                          partition_tokens=64)
    torch.cuda.synchronize()
    kp, vp = host_bits(r.kc), host_bits(r.vc)
    tables = w.block_tables.copy()
    tables[1, j:-1] = w.block_tables[1, j + 1:]
    lens = w.seq_lens.copy()
    lens[1] -= B
    ref = oracle.paged_multi_token_attention(w.q, w.q_start, kp, vp, tables, lens, w.scale)
    check_attention(w, host_f64(out), ref)
    check_attention(w, host_f64(out_p), ref)


def test_library_choice_between_the_kernels_gives_the_same_rule():
    # enough rows and work-groups for the library to pick the unpartitioned
    # kernel with partition_tokens = 0; the partitioned kernel on the same
    # input agrees within the tolerance, and both match the oracle
    w = pi.make_workload(3, S=24, len_lo=100, len_hi=600, seed=32, q_lens=16)
    announce(f"library choice: {w.S} sequences x 16 rows, G={w.G}")
    r = MRun(w, partition_tokens=0)
    full_check(w, r)
    m = pkv()
    out_p = m.paged_multi_token_attention(r.q, r.qs, w.max_q_len, r.kc, r.vc, r.bt, r.sl, w.scale,
                                          partition_tokens=512)
    torch.cuda.synchronize()
    d = (out_p.float() - r.out.float()).abs().max().item()
    announce(f"  partitioned vs library's choice: max difference {d:.3g}")
    assert d <= 4e-3


@pytest.mark.parametrize("dtype,B", [("bf16", 16), ("bf16", 1), ("bf16", 8), ("bf16", 32), ("bf16", 64), ("f32", 16),
                                     ("f32", 64), ("fp8", 16), ("fp8", 64)])
def test_block_wise_append_equals_the_slot_append(dtype, B):
    # pkv_multi_token_append against kv_cache_append through the rows' slot
    # mapping: whole pools bit-identical, and equal to the oracle's pools;
    # also with a block ID outside the pool and lengths shortened below the
    # row count (rows at negative positions are skipped by both)
    w = pi.make_workload(3, S=5, len_lo=20, len_hi=400, dtype=dtype, B=B, seed=33, q_lens=None)
    q_lens = np.minimum([1, 70, 17, 130, 5], w.seq_lens)
    w = pi.make_workload(3, S=5, len_lo=20, len_hi=400, dtype=dtype, B=B, seed=33, q_lens=q_lens)
    announce(f"block-wise append {dtype} B={B}: lens={list(w.seq_lens)} q_start={list(w.q_start)}")
    m = pkv()
    sc = dict(k_scale=w.k_scale, v_scale=w.v_scale)
    bt, qs = dev(w.block_tables), dev(w.q_start)
    nk, nv = dev(w.new_k), dev(w.new_v)
    for variant in ("plain", "bad block", "short"):
        sl = dev(w.seq_lens)
        if variant == "bad block":
            bt = dev(w.block_tables)
            bt[3, 1] = w.num_blocks + 7
        if variant == "short":
            sl = sl - 3
        kc1, vc1 = dev(w.k_cache), dev(w.v_cache)
        kc2, vc2 = dev(w.k_cache), dev(w.v_cache)
        slots = m.multi_token_slot_mapping(bt, sl, qs, w.rows, w.max_q_len, w.B)
        m.kv_cache_append(nk, nv, slots, kc1, vc1, **sc)
        m.multi_token_append(nk, nv, qs, w.max_q_len, bt, sl, kc2, vc2, **sc)
        torch.cuda.synchronize()
        assert same_bytes(host_bits(kc2), host_bits(kc1)), variant
        assert same_bytes(host_bits(vc2), host_bits(vc1)), variant
        if variant == "plain":
            ref_slots, kp, vp, _ = oracle.multi_token_step(w)
            assert same_bytes(host_bits(kc2), kp)
            assert same_bytes(host_bits(vc2), vp)


@pytest.mark.parametrize("dtype,hs,B,Hq,Hkv", [
    ("bf16", 64, 16, 8, 8), ("bf16", 64, 32, 16, 2), ("bf16", 64, 64, 4, 4), ("bf16", 128, 16, 16, 1),
    ("bf16", 128, 32, 12, 4), ("fp8", 64, 16, 8, 2), ("fp8", 128, 64, 16, 2), ("fp8", 64, 32, 4, 4),
])
def test_unpartitioned_kernel_shapes(dtype, hs, B, Hq, Hkv):
    w0 = pi.make_workload(3, S=4, len_lo=1, len_hi=900, dtype=dtype, hs=hs, B=B, Hq=Hq, Hkv=Hkv, seed=34)
    q_lens = np.minimum([3, 70, 200, 1], w0.seq_lens)
    w = pi.make_workload(3, S=4, len_lo=1, len_hi=900, dtype=dtype, hs=hs, B=B, Hq=Hq, Hkv=Hkv, seed=34,
                         q_lens=q_lens)
    announce(f"unpartitioned {dtype} hs={hs} B={B} Hq={Hq} Hkv={Hkv} lens={list(w.seq_lens)} q_start={list(w.q_start)}")
    full_check(w, MRun(w, partition_tokens=pkv().PARTITION_NONE))


# Longest-first schedule of a multi-token batch: written by the slot mapping
# launch (as the decode append writes it) and read by the partitioned
# attention, in rank order below 65 sequences and through the chunk list
# (one work-group per listed chunk, KV head and row tile) above.  Results
# must not depend on it.
@pytest.mark.parametrize("S,q_lens", [(48, 4), (80, 4), (80, 9), (72, 1)])
def test_step_with_schedule_bit_identical_to_the_separate_calls(S, q_lens):
    w = pi.make_workload(3, S=S, len_lo=16, len_hi=3000, q_lens=q_lens)
    announce(f"multi-token step with schedule: S={S} q_lens={q_lens} rows={w.rows} max_len={int(w.seq_lens.max())}")
    r = MRun(w)
    m = pkv()
    ws = m.alloc_multi_token_step_workspace(r.q, r.kc, r.vc, r.bt, w.max_q_len)
    plain = m.alloc_multi_token_workspace(r.q, r.kc, r.vc, r.bt, w.max_q_len)
    assert ws is not None and ws.numel() > (plain.numel() if plain is not None else 0)
    kc, vc = dev(w.k_cache), dev(w.v_cache)
    slots = torch.empty(w.rows, dtype=torch.int64, device="cuda")
    out = m.paged_multi_token_step(r.q, r.nk, r.nv, kc, vc, r.qs, w.max_q_len, r.bt, r.sl, w.scale,
                                   slot_mapping=slots, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(slots, r.slots)
    assert torch.equal(kc.view(torch.int16), r.kc.view(torch.int16))
    assert torch.equal(vc.view(torch.int16), r.vc.view(torch.int16))
    assert torch.equal(out.view(torch.int16), r.out.view(torch.int16))


def test_step_with_schedule_matches_the_oracle():
    w = pi.make_workload(3, S=70, len_lo=16, len_hi=2600, q_lens=6)
    announce(f"multi-token step with schedule vs oracle: S=70 rows={w.rows}")
    m = pkv()
    q, kc, vc = dev(w.q), dev(w.k_cache), dev(w.v_cache)
    bt, sl, qs = dev(w.block_tables), dev(w.seq_lens), dev(w.q_start)
    slots = torch.empty(w.rows, dtype=torch.int64, device="cuda")
    out = m.paged_multi_token_step(q, dev(w.new_k), dev(w.new_v), kc, vc, qs, w.max_q_len, bt, sl, w.scale,
                                   slot_mapping=slots)
    torch.cuda.synchronize()
    full_check(w, SimpleNamespace(slots=slots, kc=kc, vc=vc, out=out))


@pytest.mark.parametrize("S", [40, 90])
def test_attention_with_a_caller_schedule(S):
    # multi_token_slot_mapping writes the same schedule bytes as the decode
    # append for the same tables and lengths, and the stand-alone attention
    # gives the same bits with it as without it
    w = pi.make_workload(3, S=S, len_lo=16, len_hi=3000, q_lens=3)
    announce(f"multi-token attention with a caller schedule: S={S}")
    r = MRun(w)
    m = pkv()
    sched = m.alloc_schedule(r.bt).zero_()  # zeroed: the padding is compared too
    slots = m.multi_token_slot_mapping(r.bt, r.sl, r.qs, w.rows, w.max_q_len, w.B, schedule=sched)
    out = m.paged_multi_token_attention(r.q, r.qs, w.max_q_len, r.kc, r.vc, r.bt, r.sl, w.scale, schedule=sched)
    dsched = m.alloc_schedule(r.bt).zero_()
    kc, vc = dev(w.k_cache), dev(w.v_cache)
    m.decode_append(r.nk[:S].contiguous(), r.nv[:S].contiguous(), r.bt, r.sl, kc, vc, schedule=dsched)
    torch.cuda.synchronize()
    assert torch.equal(slots, r.slots)
    assert torch.equal(out.view(torch.int16), r.out.view(torch.int16))
    assert torch.equal(sched, dsched)


@pytest.mark.parametrize("S,q_lens,B", [(20, 40, 16), (13, 70, 32), (9, [200, 3, 64, 17, 90, 1, 33, 129, 8], 64)])
def test_unpartitioned_kernel_with_the_schedule(S, q_lens, B):
    # the unpartitioned kernel takes (sequence, KV head) pairs longest first
    # when given the schedule (13 sequences x 8 KV heads is not a whole round
    # of 8 pairs per XCD): the step with its schedule, the attention with a
    # caller schedule and the attention without one give the same bits, and
    # match the oracle
    w = pi.make_workload(3, S=S, len_lo=16, len_hi=2000, B=B, seed=40 + S, q_lens=q_lens)
    announce(f"unpartitioned kernel with schedule: S={S} B={B} rows={w.rows} lens {list(w.seq_lens)}")
    m = pkv()
    NONE = m.PARTITION_NONE
    r = MRun(w, partition_tokens=NONE)
    full_check(w, r)
    ws = m.alloc_multi_token_step_workspace(r.q, r.kc, r.vc, r.bt, w.max_q_len, NONE)
    assert ws is not None
    kc, vc = dev(w.k_cache), dev(w.v_cache)
    slots = torch.empty(w.rows, dtype=torch.int64, device="cuda")
    out = m.paged_multi_token_step(r.q, r.nk, r.nv, kc, vc, r.qs, w.max_q_len, r.bt, r.sl, w.scale,
                                   slot_mapping=slots, workspace=ws, partition_tokens=NONE)
    sched = m.alloc_schedule(r.bt)
    m.multi_token_slot_mapping(r.bt, r.sl, r.qs, w.rows, w.max_q_len, w.B, schedule=sched)
    out2 = m.paged_multi_token_attention(r.q, r.qs, w.max_q_len, r.kc, r.vc, r.bt, r.sl, w.scale,
                                         partition_tokens=NONE, schedule=sched)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), r.out.view(torch.int16))
    assert torch.equal(out2.view(torch.int16), r.out.view(torch.int16))


def test_unpartitioned_kernel_contains_a_foreign_schedule():
    # a schedule never written for this batch (every word outside it): no
    # work-group writes outside out (guard rows around it keep their bits)
    w = pi.make_workload(3, S=10, len_lo=100, len_hi=900, seed=50, q_lens=70)
    announce("unpartitioned kernel, foreign schedule")
    m = pkv()
    q, kc, vc = dev(w.q), dev(w.k_cache), dev(w.v_cache)
    bt, sl, qs = dev(w.block_tables), dev(w.seq_lens), dev(w.q_start)
    sched = m.alloc_schedule(bt)
    sched.view(torch.int32).fill_(0x7FFF7FFF)
    guard = torch.full((w.rows + 2, w.Hq, w.hs), 7.0, dtype=torch.bfloat16, device="cuda")
    out = guard[1:w.rows + 1]
    m.paged_multi_token_attention(q, qs, w.max_q_len, kc, vc, bt, sl, w.scale, out=out,
                                  partition_tokens=m.PARTITION_NONE, schedule=sched)
    torch.cuda.synchronize()
    assert torch.all(guard[0] == 7.0).item() and torch.all(guard[w.rows + 1] == 7.0).item()


@pytest.mark.parametrize("P", [0, 64, -1])
def test_broken_row_ranges_are_contained(P):
    # caller contract violations the kernels must contain (both kernels):
    # a sequence whose rows run past num_q_rows is skipped, rows past
    # max_q_len are not computed, rows at a negative position (n > L) get
    # zeros; the other sequences' rows equal those of a valid call
    w = pi.make_workload(3, S=3, seq_lens=[500, 300, 200], q_lens=[3, 4, 2])
    announce(f"broken row ranges, partition_tokens={P}")
    m = pkv()
    q, kc, vc, bt, sl = dev(w.q), dev(w.k_cache), dev(w.v_cache), dev(w.block_tables), dev(w.seq_lens)
    qs_ok = dev(w.q_start)  # [0, 3, 7, 9]
    ref = m.paged_multi_token_attention(q, qs_ok, w.max_q_len, kc, vc, bt, sl, w.scale, partition_tokens=P)
    sentinel = 7.0

    def run(q_start, max_q_len, lens):
        out = torch.full_like(q, sentinel)
        return m.paged_multi_token_attention(q, dev(np.array(q_start, np.int32)), max_q_len, kc, vc, bt,
                                             dev(np.array(lens, np.int32)), w.scale, out=out, partition_tokens=P)

    lens = [int(x) for x in w.seq_lens]
    # sequence 2's rows end past num_q_rows = 9: skipped
    a = run([0, 3, 7, 12], w.max_q_len, lens)
    # max_q_len 3 < sequence 1's 4 rows: its 4th row is not computed
    b = run([0, 3, 7, 9], 3, lens)
    # sequence 1 holds 2 tokens for its 4 rows: rows at positions -2, -1 get zeros
    c = run([0, 3, 7, 9], w.max_q_len, [lens[0], 2, lens[2]])
    torch.cuda.synchronize()
    eq = lambda x, y: torch.equal(x.view(torch.int16), y.view(torch.int16))
    assert eq(a[:7], ref[:7]) and torch.all(a[7:].float() == sentinel)
    assert eq(b[:3], ref[:3]) and eq(b[7:], ref[7:]) and torch.all(b[6].float() == sentinel)
    assert eq(c[:3], ref[:3]) and eq(c[7:], ref[7:]) and torch.all(c[3:5].float() == 0)
    assert torch.isfinite(c[5:7].float()).all()
