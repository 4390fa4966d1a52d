"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Inputs come from the seeded generators; parity-mode pools hold NaN in every
slot that carries no data, so a read outside the sequence shows up.  Bars:
slot mapping and append bit-exact (whole pools compared); attention max-abs
error <= 1e-5 (fp32) and <= 2e-3 (bf16) against the fp64 oracle.
Small variants and the full-size configurations (in the launch
configuration the benchmark times) are compared element by element, every
(sequence, query head) row.  Every bf16 configuration also runs with an fp32
output: that output is held to the fp32 bar (the kernel's own error, apart
from the output rounding), and the bf16 output of the same call must be
exactly its round-to-nearest-even.
"""
import numpy as np
import pytest

import oracle
import pkv_inputs as pi

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-3, "fp8": 2e-3}  # fp8 pools: bf16 outputs


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_35_amd as pkv

    pkv.library()  # fails loudly when the HIP library is missing
    torch.cuda.set_device(0)


def pkv():
    import paged_kv_cache_35_amd as m

    return m


def dev(a):
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host_bits(t):
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def same_bytes(a, b):
    a = np.ascontiguousarray(a)
    b = np.ascontiguousarray(b)
    return a.shape == b.shape and np.array_equal(a.reshape(-1).view(np.uint8), b.reshape(-1).view(np.uint8))


def host_f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def announce(msg):
    print(msg, flush=True)


class Run:
    def __init__(self, w, partition_tokens=None):
        self.w = w
        P = w.partition_tokens if partition_tokens is None else partition_tokens
        self.q, self.kc, self.vc = dev(w.q), dev(w.k_cache), dev(w.v_cache)
        self.bt, self.sl = dev(w.block_tables), dev(w.seq_lens)
        self.nk, self.nv = dev(w.new_k), dev(w.new_v)
        m = pkv()
        self.slots = m.decode_slot_mapping(self.bt, self.sl, w.B)
        m.kv_cache_append(self.nk, self.nv, self.slots, self.kc, self.vc)
        self.out = m.paged_decode_attention(self.q, self.kc, self.vc, self.bt, self.sl, w.scale,
                                            partition_tokens=P)
        torch.cuda.synchronize()

    def attend_again(self, partition_tokens=0, block_tables=None):
        m = pkv()
        out = m.paged_decode_attention(self.q, self.kc, self.vc, self.bt if block_tables is None else block_tables,
                                       self.sl, self.w.scale, partition_tokens=partition_tokens)
        torch.cuda.synchronize()
        return out


def bf16_ulp(x):
    """Spacing of bfloat16 numbers at magnitude |x| (8 significant bits)."""
    e = np.floor(np.log2(np.maximum(np.abs(x), np.finfo(np.float32).tiny)))
    return np.exp2(e - 7)


def check_attention(w, got, ref, out_f32=False):
    """Max-abs error within the tolerance.  A bf16 output of magnitude >= 1 can
    be off by half a bf16 ulp from rounding alone (more than 2e-3), so those
    elements are held to half a bf16 ulp of the oracle plus 1e-5 relative
    (round to nearest even of a result within fp32 accumulation error), and
    reported.  out_f32: an fp32 output of a bf16 call, held to the fp32 bar."""
    tol = TOL["f32"] if out_f32 else TOL[w.dtype]
    assert np.isfinite(got).all(), "non-finite output"
    diff = np.abs(got - ref)
    if w.dtype in ("bf16", "fp8") and not out_f32:  # bf16 outputs
        big = np.abs(ref) >= 1.0
        if big.any():
            bar = 0.5 * bf16_ulp(ref[big]) + 1e-5 * np.abs(ref[big])
            announce(f"  {int(big.sum())} outputs with |out| >= 1 held to half a bf16 ulp + 1e-5 relative; "
                     f"worst error / half ulp {float((diff[big] / (0.5 * bf16_ulp(ref[big]))).max()):.3f}")
            assert (diff[big] <= bar).all()
        diff = np.where(big, 0.0, diff)
    err = float(diff.max()) if diff.size else 0.0
    announce(f"  max abs error {err:.3g} (tolerance {tol}{', fp32 output' if out_f32 else ''})")
    assert err <= tol


def bf16_rne_bits(x32):
    """bfloat16 bit patterns of float32 values, rounded to nearest even (finite inputs)."""
    b = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


def check_rounding(out_bf16, out_f32):
    """The bf16 output of a call is exactly the round-to-nearest-even of the
    fp32 output of the same call."""
    want = bf16_rne_bits(out_f32.float().cpu().numpy())
    got = host_bits(out_bf16)
    bad = int((got != want).sum())
    announce(f"  bf16 output == RNE(fp32 output): {got.size - bad}/{got.size} elements")
    assert bad == 0


SMALL = {
    1: dict(),
    2: dict(S=6, len_lo=128, len_hi=700),
    3: dict(S=12, len_lo=16, len_hi=1500),
    4: dict(S=2, len_lo=1500, len_hi=5000),
    5: dict(S=8, len_hi=256),
}


def check_fp32_output(w, r, ref, partition_tokens=None):
    """bf16 configurations: the same attention call with an fp32 output is
    within the fp32 bar of the oracle, and r.out is its exact rounding."""
    if w.dtype == "f32":
        return
    P = w.partition_tokens if partition_tokens is None else partition_tokens
    out32 = pkv().paged_decode_attention(r.q, r.kc, r.vc, r.bt, r.sl, w.scale, partition_tokens=P,
                                         out_dtype=torch.float32)
    torch.cuda.synchronize()
    check_attention(w, host_f64(out32), ref, out_f32=True)
    check_rounding(r.out, out32)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_small_config_full_parity(cfg):
    w = pi.make_workload(cfg, **SMALL[cfg])
    announce(f"small config {cfg}: S={w.S} lens={list(w.seq_lens)} dtype={w.dtype} G={w.G} B={w.B}")
    r = Run(w)
    slots, kp, vp, ref = oracle.decode_step(w)
    assert np.array_equal(r.slots.cpu().numpy(), slots)
    assert same_bytes(host_bits(r.kc), kp)
    assert same_bytes(host_bits(r.vc), vp)
    check_attention(w, host_f64(r.out), ref)
    check_fp32_output(w, r, ref)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_full_config_parity(cfg):
    w = pi.make_workload(cfg)
    announce(f"full config {cfg}: S={w.S} Hq={w.Hq} Hkv={w.Hkv} blocks={w.num_blocks} sumL={int(w.seq_lens.sum())}")
    r = Run(w)
    slots = oracle.decode_slot_mapping(w.block_tables, w.seq_lens, w.B)
    assert np.array_equal(r.slots.cpu().numpy(), slots)
    kp, vp = w.k_cache.copy(), w.v_cache.copy()
    oracle.kv_append(w.new_k, w.new_v, slots, kp, vp)
    assert same_bytes(host_bits(r.kc), kp), "key pool differs after append"
    assert same_bytes(host_bits(r.vc), vp), "value pool differs after append"
    # every (sequence, query head) row against the oracle's full pass
    ref = oracle.paged_attention(w.q, kp, vp, w.block_tables, w.seq_lens, w.scale)
    check_attention(w, host_f64(r.out), ref)
    check_fp32_output(w, r, ref)
    # every output row is finite (NaN-poisoned slots never leak)
    assert torch.isfinite(r.out.float()).all().item()


@pytest.mark.parametrize("dtype,hs,B,Hq,Hkv", [
    ("f32", 64, 16, 8, 8), ("f32", 128, 32, 8, 2), ("f32", 64, 32, 16, 1), ("f32", 128, 16, 4, 4),
    ("bf16", 64, 16, 8, 8), ("bf16", 64, 32, 16, 2), ("bf16", 128, 16, 16, 1), ("bf16", 128, 32, 12, 4),
    ("bf16", 128, 16, 2, 2), ("bf16", 64, 16, 24, 8),
])
def test_shape_sweep(dtype, hs, B, Hq, Hkv):
    w = pi.make_workload(3, S=7, len_lo=1, len_hi=1300, dtype=dtype, hs=hs, B=B, Hq=Hq, Hkv=Hkv)
    announce(f"shape sweep {dtype} hs={hs} B={B} Hq={Hq} Hkv={Hkv} lens={list(w.seq_lens)}")
    r = Run(w)
    ref = oracle.decode_step(w)[3]
    check_attention(w, host_f64(r.out), ref)


def test_edge_lengths():
    # L = 1, exactly one block, a block plus one token, the table's maximum,
    # and an empty sequence (zero output)
    B = 16
    lens = [1, B, B + 1, 2 * B - 1, 64 * B, 3, 64 * B - 1, 0]
    w = pi.make_workload(2, seq_lens=lens)
    announce(f"edge lengths {lens} M={w.M}")
    r = Run(w)
    ref = oracle.decode_step(w)[3]
    got = host_f64(r.out)
    assert np.all(got[7] == 0)
    check_attention(w, got, ref)
    assert r.slots.cpu().numpy()[7] == -1


@pytest.mark.parametrize("S", [64, 65])
def test_batch_sizes_around_the_in_kernel_ranking_limit(S):
    # a stand-alone attention call ranks batches of up to 64 sequences itself
    # and attends larger ones in batch order (lengths up to 2600 tokens:
    # some sequences span two chunks)
    w = pi.make_workload(3, S=S, len_lo=1, len_hi=2600)
    announce(f"batch of {S} sequences, lengths {int(w.seq_lens.min())}..{int(w.seq_lens.max())}")
    r = Run(w)
    ref = oracle.decode_step(w)[3]
    check_attention(w, host_f64(r.out), ref)


def test_schedule_does_not_change_results():
    # the same 64 sequences attended as a batch of 64 (ranked in the kernel),
    # as the first 64 of a batch of 65 (batch order), and with the schedule
    # written by the append launch: identical bits
    w = pi.make_workload(3, S=64, len_lo=1, len_hi=2600)
    announce("longest-first (in kernel, from the append) vs batch order")
    r = Run(w)
    m = pkv()
    bt = torch.cat([r.bt, r.bt[:1]])
    sl = torch.cat([r.sl, torch.zeros(1, dtype=torch.int32, device="cuda")])
    q = torch.cat([r.q, r.q[:1]])
    out = m.paged_decode_attention(q, r.kc, r.vc, bt, sl, w.scale)
    sched = m.alloc_schedule(r.bt)
    kc, vc = dev(w.k_cache), dev(w.v_cache)
    m.decode_append(r.nk, r.nv, r.bt, r.sl, kc, vc, schedule=sched)
    out2 = m.paged_decode_attention(r.q, kc, vc, r.bt, r.sl, w.scale, schedule=sched)
    torch.cuda.synchronize()
    assert torch.equal(out[:64].view(torch.int16), r.out.view(torch.int16))
    assert torch.all(out[64].float() == 0)
    assert torch.equal(out2.view(torch.int16), r.out.view(torch.int16))


def expected_schedule(block_tables, seq_lens, B):
    """Longest-first order by blocks (ties by index), written out on the host."""
    M = block_tables.shape[1]
    L = np.clip(seq_lens.astype(np.int64), 0, M * B)
    blocks = (L + B - 1) // B
    order = sorted(range(len(L)), key=lambda i: (-int(blocks[i]), i))
    return np.array(order, np.int32), seq_lens[order].astype(np.int32), block_tables[order].astype(np.int32)


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_schedule_contents(cfg):
    w = pi.make_workload(cfg, **SMALL[cfg])
    S = w.S
    announce(f"schedule contents config {cfg}: lens={list(w.seq_lens)}")
    m = pkv()
    kc, vc = dev(w.k_cache), dev(w.v_cache)
    bt, sl = dev(w.block_tables), dev(w.seq_lens)
    sched = m.alloc_schedule(bt)
    m.decode_append(dev(w.new_k), dev(w.new_v), bt, sl, kc, vc, schedule=sched)
    torch.cuda.synchronize()
    raw = sched.cpu().numpy().view(np.int32)
    vec = -(-S * 4 // 16) * 4  # ints per rounded vector
    order, lens, tables = expected_schedule(w.block_tables, w.seq_lens, w.B)
    assert np.array_equal(raw[:S], order)
    assert np.array_equal(raw[vec:vec + S], lens)
    assert np.array_equal(raw[2 * vec:2 * vec + S * w.M].reshape(S, w.M), tables)
    # the chunk list of the default partitioning (CB = 4 partitions of
    # min(512 tokens, 64 blocks, the table) each): every full chunk (CB
    # blocks) by sequence index, then the partial chunks (blocks % CB, or an
    # empty sequence's one chunk) by decreasing size, ties by index
    P = min(512, 64 * w.B, w.M * w.B)
    CB = (P // w.B) * 4
    L = np.clip(w.seq_lens.astype(np.int64), 0, w.M * w.B)
    blocks = -(-L // w.B)
    rank = {int(s): y for y, s in enumerate(order)}
    full = [(rank[s] | (c << 16), s) for s in range(S) for c in range(int(blocks[s] // CB))]
    parts = [(-(int(blocks[s] % CB)), s) for s in range(S) if blocks[s] % CB or blocks[s] == 0]
    items = full + [(rank[s] | (int(blocks[s] // CB) << 16), s) for _, s in sorted(parts)]
    base = 2 * vec + -(-S * w.M // 4) * 4
    assert raw[base] == len(items)
    got = raw[base + 4:base + 4 + 2 * len(items)].view(np.uint32).reshape(-1, 2)
    assert np.array_equal(got, np.array(items, np.uint32).reshape(-1, 2))


@pytest.mark.parametrize("S", [4096, 4097])
def test_step_batch_sizes_around_the_schedule_limit(S):
    # the decode step schedules up to 4096 sequences and attends larger
    # batches in batch order
    w = pi.make_workload(2, S=S, len_lo=1, len_hi=40, hs=64, Hq=2, Hkv=2)
    announce(f"decode step, batch of {S}, lengths 1..40, 2 heads of 64")
    out, kc, vc, slots = run_step(w)
    ref_slots, kp, vp, ref = oracle.decode_step(w)
    assert np.array_equal(slots.cpu().numpy(), ref_slots)
    assert same_bytes(host_bits(kc), kp)
    assert same_bytes(host_bits(vc), vp)
    check_attention(w, host_f64(out), ref)


@pytest.mark.parametrize("P", [16, 32, 256, 512, 1024])
def test_partition_length_sweep(P):
    w = pi.make_workload(3, S=5, len_lo=16, len_hi=4000)
    announce(f"partition sweep P={P} lens={list(w.seq_lens)}")
    r = Run(w, partition_tokens=P)
    ref = oracle.decode_step(w)[3]
    check_attention(w, host_f64(r.out), ref)


def test_repeat_runs_bit_identical():
    w = pi.make_workload(4, S=2, len_lo=3000, len_hi=9000)
    announce("determinism: repeated calls")
    r = Run(w)
    a = r.out.clone()
    for _ in range(3):
        b = r.attend_again(partition_tokens=w.partition_tokens)
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("S", [12, 80, 300])
def test_schedule_reused_by_repeated_attention_calls(S):
    # A schedule is read, never consumed, by the attention launch: calls
    # that reuse one schedule without a new append, and calls of two batches
    # with their own schedules in between, all give the same bits as the
    # first call, and the oracle's result.  S = 12 walks the ranked grid,
    # S = 80 and 300 the chunk list (lengths up to 3000: two chunks for the
    # long sequences, so the chunk merge runs too).
    m = pkv()
    runs = []
    for k, n in enumerate((S, S + 7)):
        w = pi.make_workload(3, S=n, len_lo=1, len_hi=3000, seed=100 + k)
        q, kc, vc = dev(w.q), dev(w.k_cache), dev(w.v_cache)
        bt, sl = dev(w.block_tables), dev(w.seq_lens)
        sched = m.alloc_schedule(bt)
        m.decode_append(dev(w.new_k), dev(w.new_v), bt, sl, kc, vc, schedule=sched)
        runs.append((w, q, kc, vc, bt, sl, sched))
    announce(f"schedule reused: batches of {S} and {S + 7}, three calls each, interleaved")
    firsts = []
    for rep in range(3):
        for i, (w, q, kc, vc, bt, sl, sched) in enumerate(runs):
            out = m.paged_decode_attention(q, kc, vc, bt, sl, w.scale, schedule=sched)
            torch.cuda.synchronize()
            if rep == 0:
                firsts.append(out.clone())
                check_attention(w, host_f64(out), oracle.decode_step(w)[3])
            else:
                assert torch.equal(out.view(torch.int16), firsts[i].view(torch.int16)), (rep, i)


def test_block_relabelling_bit_identical():
    w = pi.make_workload(3, S=9, len_lo=16, len_hi=2500)
    announce("determinism: relabelled physical blocks")
    a = Run(w).out
    b = Run(pi.relabel_blocks(w, 5)).out
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_shared_prefix_bit_identical_to_copies():
    w = pi.make_workload(5, S=10, len_hi=512)
    announce("determinism: shared prefix vs private copies")
    a = Run(w).out
    b = Run(pi.unshare_blocks(w)).out
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_append_skips_negative_slots_and_leaves_the_rest():
    w = pi.make_workload(2, S=6, len_lo=20, len_hi=90)
    announce("append with skipped slots")
    kc, vc = dev(w.k_cache), dev(w.v_cache)
    slots = oracle.decode_slot_mapping(w.block_tables, w.seq_lens, w.B)
    slots[[1, 4]] = -1
    pkv().kv_cache_append(dev(w.new_k), dev(w.new_v), dev(slots), kc, vc)
    torch.cuda.synchronize()
    kp, vp = w.k_cache.copy(), w.v_cache.copy()
    oracle.kv_append(w.new_k, w.new_v, slots, kp, vp)
    assert same_bytes(host_bits(kc), kp)
    assert same_bytes(host_bits(vc), vp)


@pytest.mark.parametrize("cfg", [1, 2, 4, 5])
def test_decode_append_bit_exact(cfg):
    w = pi.make_workload(cfg, **SMALL[cfg])
    announce(f"decode append config {cfg}: lens={list(w.seq_lens)}")
    kc, vc = dev(w.k_cache), dev(w.v_cache)
    slots = torch.full((w.S,), -7, dtype=torch.int64, device="cuda")
    pkv().decode_append(dev(w.new_k), dev(w.new_v), dev(w.block_tables), dev(w.seq_lens), kc, vc, slot_mapping=slots)
    torch.cuda.synchronize()
    ref_slots = oracle.decode_slot_mapping(w.block_tables, w.seq_lens, w.B)
    kp, vp = w.k_cache.copy(), w.v_cache.copy()
    oracle.kv_append(w.new_k, w.new_v, ref_slots, kp, vp)
    assert np.array_equal(slots.cpu().numpy(), ref_slots)
    assert same_bytes(host_bits(kc), kp)
    assert same_bytes(host_bits(vc), vp)


def test_decode_append_skips_empty_sequences():
    lens = [5, 0, 17, 0, 1]
    w = pi.make_workload(2, seq_lens=lens)
    announce(f"decode append with empty sequences {lens}")
    kc, vc = dev(w.k_cache), dev(w.v_cache)
    pkv().decode_append(dev(w.new_k), dev(w.new_v), dev(w.block_tables), dev(w.seq_lens), kc, vc)
    torch.cuda.synchronize()
    ref_slots = oracle.decode_slot_mapping(w.block_tables, w.seq_lens, w.B)
    assert list(ref_slots[[1, 3]]) == [-1, -1]
    kp, vp = w.k_cache.copy(), w.v_cache.copy()
    oracle.kv_append(w.new_k, w.new_v, ref_slots, kp, vp)
    assert same_bytes(host_bits(kc), kp)
    assert same_bytes(host_bits(vc), vp)


def run_step(w, partition_tokens=None):
    P = w.partition_tokens if partition_tokens is None else partition_tokens
    q, kc, vc = dev(w.q), dev(w.k_cache), dev(w.v_cache)
    bt, sl = dev(w.block_tables), dev(w.seq_lens)
    slots = torch.full((w.S,), -7, dtype=torch.int64, device="cuda")
    out = pkv().paged_decode_step(q, dev(w.new_k), dev(w.new_v), kc, vc, bt, sl, w.scale, slot_mapping=slots,
                                  partition_tokens=P)
    torch.cuda.synchronize()
    return out, kc, vc, slots


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_step_matches_oracle(cfg):
    w = pi.make_workload(cfg, **SMALL[cfg])
    announce(f"decode step config {cfg}: lens={list(w.seq_lens)}")
    out, kc, vc, slots = run_step(w)
    ref_slots, kp, vp, ref = oracle.decode_step(w)
    assert np.array_equal(slots.cpu().numpy(), ref_slots)
    assert same_bytes(host_bits(kc), kp)
    assert same_bytes(host_bits(vc), vp)
    check_attention(w, host_f64(out), ref)


@pytest.mark.parametrize("cfg,P", [(1, None), (2, None), (3, None), (3, 256), (4, None), (4, 0), (5, None)])
def test_step_bit_identical_to_append_then_attention(cfg, P):
    w = pi.make_workload(cfg, **SMALL[cfg])
    announce(f"decode step vs separate launches, config {cfg}, P={P}")
    out, kc, vc, slots = run_step(w, P)
    r = Run(w, partition_tokens=P)
    bits = torch.int16 if out.dtype == torch.bfloat16 else torch.int32
    assert torch.equal(out.view(bits), r.out.view(bits))
    assert torch.equal(kc.view(torch.int16), r.kc.view(torch.int16))
    assert torch.equal(vc.view(torch.int16), r.vc.view(torch.int16))
    assert torch.equal(slots, r.slots)


def test_step_edge_lengths():
    B = 16
    lens = [1, B, B + 1, 64 * B, 0, 3, 64 * B - 1, 2 * B]
    w = pi.make_workload(2, seq_lens=lens)
    announce(f"decode step edge lengths {lens}")
    out, kc, vc, slots = run_step(w)
    ref_slots, kp, vp, ref = oracle.decode_step(w)
    assert np.array_equal(slots.cpu().numpy(), ref_slots)
    assert same_bytes(host_bits(kc), kp)
    assert same_bytes(host_bits(vc), vp)
    got = host_f64(out)
    assert np.all(got[4] == 0)
    check_attention(w, got, ref)


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_step_full_config(cfg):
    w = pi.make_workload(cfg)
    announce(f"decode step, full config {cfg}")
    out, kc, vc, slots = run_step(w)
    ref_slots = oracle.decode_slot_mapping(w.block_tables, w.seq_lens, w.B)
    assert np.array_equal(slots.cpu().numpy(), ref_slots)
    kp, vp = w.k_cache.copy(), w.v_cache.copy()
    oracle.kv_append(w.new_k, w.new_v, ref_slots, kp, vp)
    assert same_bytes(host_bits(kc), kp)
    assert same_bytes(host_bits(vc), vp)
    ref = oracle.paged_attention(w.q, kp, vp, w.block_tables, w.seq_lens, w.scale)
    check_attention(w, host_f64(out), ref)
    assert torch.isfinite(out.float()).all().item()
    # the step with an fp32 output (the pools already hold the new tokens:
    # a second append rewrites the same bits)
    out32 = pkv().paged_decode_step(dev(w.q), dev(w.new_k), dev(w.new_v), kc, vc, dev(w.block_tables),
                                    dev(w.seq_lens), w.scale, partition_tokens=w.partition_tokens,
                                    out_dtype=torch.float32)
    torch.cuda.synchronize()
    check_attention(w, host_f64(out32), ref, out_f32=True)
    check_rounding(out, out32)


@pytest.mark.parametrize("cfg", [2, 3])
def test_lengths_outside_the_table_are_clamped(cfg):
    # caller contract violations the kernels must contain: a length above
    # max_blocks_per_seq * B reads the whole table row (as that maximum), a
    # negative length reads nothing (zero output); bit-identical to the
    # clamped lengths, with and without a schedule, and the step's append
    # skips both (slot -1)
    w = pi.make_workload(cfg, S=6, len_lo=40, len_hi=300)
    cap = w.M * w.B
    announce(f"lengths outside the table: config {cfg} M={w.M} B={w.B}")
    m = pkv()
    q, kc, vc, bt = dev(w.q), dev(w.k_cache), dev(w.v_cache), dev(w.block_tables)
    bad = w.seq_lens.copy()
    bad[1] = cap + 1000
    bad[3] = -7
    clamped = np.clip(bad, 0, cap).astype(np.int32)
    sl_bad, sl_ok = dev(bad.astype(np.int32)), dev(clamped)
    ref = m.paged_decode_attention(q, kc, vc, bt, sl_ok, w.scale)
    got = m.paged_decode_attention(q, kc, vc, bt, sl_bad, w.scale)
    sched = m.alloc_schedule(bt)
    kc2, vc2 = kc.clone(), vc.clone()
    slots = m.decode_append(dev(w.new_k), dev(w.new_v), bt, sl_bad, kc2, vc2,
                            slot_mapping=torch.empty(w.S, dtype=torch.int64, device="cuda"), schedule=sched)
    got_s = m.paged_decode_attention(q, kc, vc, bt, sl_bad, w.scale, schedule=sched)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    assert torch.equal(got_s.view(torch.int16), ref.view(torch.int16))
    assert torch.all(got[3] == 0)
    s = slots.cpu().numpy()
    assert s[1] == -1 and s[3] == -1


@pytest.mark.parametrize("S,fill", [(12, "constant"), (12, "ascending"), (80, "constant"), (80, "ascending")])
def test_foreign_schedule_is_contained(S, fill):
    # a schedule buffer that was never written for this batch (caller
    # error): every sequence index read from it that lies outside the batch
    # ends its work-group (attention) or pair (chunk merge) before any q, out
    # or q_start access; lengths are clamped and table entries outside the
    # pool skipped as always.  The call completes and nothing outside out is
    # written.  S = 12 reads the order (ranked launch), S = 80 the chunk list
    # (one-dimensional launch); lengths up to 3000 give two chunks per long
    # sequence, so the chunk merge runs too.
    w = pi.make_workload(3, S=S, len_lo=16, len_hi=3000)
    announce(f"foreign schedule: S={S} fill={fill}")
    m = pkv()
    q, kc, vc = dev(w.q), dev(w.k_cache), dev(w.v_cache)
    bt, sl = dev(w.block_tables), dev(w.seq_lens)
    sched = m.alloc_schedule(bt)
    words = sched.view(torch.int32)
    if fill == "constant":
        words.fill_(0x7FFF7FFF)
    else:  # every word at least S, so no order entry names a sequence of the batch
        words.copy_(torch.arange(S, S + words.numel(), dtype=torch.int32, device="cuda"))
    guard = torch.full((S + 2, w.Hq, w.hs), 7.0, dtype=torch.bfloat16, device="cuda")
    out = guard[1:S + 1]
    m.paged_decode_attention(q, kc, vc, bt, sl, w.scale, out=out, schedule=sched)
    torch.cuda.synchronize()
    assert torch.all(guard[0] == 7.0).item() and torch.all(guard[S + 1] == 7.0).item()
    # the same call with the right schedule still gives the oracle's result
    sched2 = m.alloc_schedule(bt)
    m.decode_append(dev(w.new_k), dev(w.new_v), bt, sl, kc, vc, schedule=sched2)
    m.paged_decode_attention(q, kc, vc, bt, sl, w.scale, out=out, schedule=sched2)
    torch.cuda.synchronize()
    assert torch.all(guard[0] == 7.0).item() and torch.all(guard[S + 1] == 7.0).item()
    check_attention(w, host_f64(out), oracle.decode_step(w)[3])
