"""The allocation-free decode step, paged_decode_step_static, through the C
ABI: against paged_decode_step with a caller workspace (outputs, pools and
slots bit for bit) and against the oracle, on two calls in a row whose second
batch is smaller (the library's device array keeps the first call's contents,
and nothing in the step may depend on them)."""
import numpy as np
import pytest

import oracle
import pkv_inputs as pi

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_35_amd as pkv

    pkv.library()  # fails loudly when the HIP library is missing
    torch.cuda.set_device(0)


def dev(a):
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def compare_one(w):
    import paged_kv_cache_35_amd as m

    need = m.step_workspace_bytes(w.S, w.Hq, w.Hkv, w.hs, w.M, w.B)
    print(f"config {w.config}: S={w.S} lengths {int(w.seq_lens.min())}..{int(w.seq_lens.max())}, "
          f"workspace {need} bytes of {m.STATIC_SCRATCH_BYTES}", flush=True)
    assert 0 < need <= m.STATIC_SCRATCH_BYTES
    q, bt, sl, nk, nv = dev(w.q), dev(w.block_tables), dev(w.seq_lens), dev(w.new_k), dev(w.new_v)
    kc_a, vc_a = dev(w.k_cache), dev(w.v_cache)
    kc_b, vc_b = dev(w.k_cache), dev(w.v_cache)
    slots_a = torch.full((w.S,), -7, dtype=torch.int64, device="cuda")
    slots_b = torch.full((w.S,), -7, dtype=torch.int64, device="cuda")
    out_a = m.paged_decode_step(q, nk, nv, kc_a, vc_a, bt, sl, w.scale, slot_mapping=slots_a)
    out_b = torch.empty_like(q)
    m.paged_decode_step_static(q, nk, nv, kc_b, vc_b, bt, sl, w.scale, out_b, slot_mapping=slots_b)
    torch.cuda.synchronize()
    assert torch.equal(bits(out_a), bits(out_b))
    assert torch.equal(slots_a, slots_b)
    assert torch.equal(bits(kc_a), bits(kc_b)) and torch.equal(bits(vc_a), bits(vc_b))
    ref = oracle.decode_step(w)[3]
    got = out_b.float().cpu().numpy().astype(np.float64)
    err = float(np.abs(got - ref)[np.abs(ref) < 1].max())
    print(f"  bit-identical to paged_decode_step; max abs error {err:.3g} against the oracle", flush=True)
    assert err <= 2e-3


def test_static_step_twice_second_smaller():
    # first call: 96 sequences (longest-first chunk list, two-chunk
    # sequences merged); second call: 2 long sequences (more chunks, the
    # work-group merge), a smaller workspace than the first call left behind
    first = pi.make_workload(3, S=96, len_lo=16, len_hi=3000)
    second = pi.make_workload(4, S=2, len_lo=12000, len_hi=20000)
    compare_one(first)
    compare_one(second)


def test_static_step_rejects_a_workspace_beyond_the_array():
    import paged_kv_cache_35_amd as m

    # 512 sequences of 64 query heads over tables of 4096 blocks need far more than the array holds
    S, Hq, M = 512, 64, 4096
    assert m.step_workspace_bytes(S, Hq, 8, 128, M, 32) > m.STATIC_SCRATCH_BYTES
    qb = torch.zeros((S, Hq, 128), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((1, 8, 16, 32, 8), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros((1, 8, 128, 32), dtype=torch.bfloat16, device="cuda")
    nk = torch.zeros((S, 8, 128), dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros((S, M), dtype=torch.int32, device="cuda")
    sl = torch.zeros((S,), dtype=torch.int32, device="cuda")
    with pytest.raises(m.PkvError, match="PKV_ERR_WORKSPACE"):
        m.paged_decode_step_static(qb, nk, nk, kc, vc, bt, sl, 0.1, torch.empty_like(qb))
