"""The decode and multi-token steps captured in a HIP graph and replayed, as
a serving loop would: every launch of a step (append with its schedule,
attention, chunk merge) takes its sizes and pointers at capture time and
allocates nothing, so the graph replays the same work.  Each replay is
checked bit for bit against the eager step, with other GPU work and
synchronizations between the replays.  (The library records no memset or
copy node: the schedule and partials are written by its own kernels.)"""
import numpy as np
import pytest

import pkv_inputs as pi
from test_gpu_parity import announce, dev, pkv

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pkv().library()
    torch.cuda.set_device(0)


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def replay_and_compare(graph, outs, refs, stream):
    for k in range(3):
        for o in outs:
            o.fill_(7)  # stale contents must be overwritten by the replay
        graph.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, refs):
            assert torch.equal(bits(o), bits(r)), f"replay {k} differs from the eager step"
        # unrelated eager work between replays
        x = torch.randn(1 << 20, device="cuda")
        (x * 2).sum().item()


@pytest.mark.parametrize("cfg,kw", [
    (2, dict(S=16, len_lo=100, len_hi=700)),
    (3, dict(S=80, len_lo=16, len_hi=3000)),   # chunk list and chunk merge
    (4, dict(S=2, len_lo=5000, len_hi=9000)),  # many chunks per sequence
])
def test_decode_step_graph_replays_match_eager(cfg, kw):
    w = pi.make_workload(cfg, **kw)
    announce(f"graph capture of the decode step: config {cfg} S={w.S} max_len={int(w.seq_lens.max())}")
    m = pkv()
    q, bt, sl, nk, nv = dev(w.q), dev(w.block_tables), dev(w.seq_lens), dev(w.new_k), dev(w.new_v)
    kc, vc = dev(w.k_cache), dev(w.v_cache)
    ws = m.alloc_step_workspace(q, kc, vc, bt, 0)
    out_ref = torch.empty_like(q)
    slots_ref = torch.empty(w.S, dtype=torch.int64, device="cuda")
    m.paged_decode_step(q, nk, nv, kc, vc, bt, sl, w.scale, out=out_ref, slot_mapping=slots_ref, workspace=ws)
    torch.cuda.synchronize()
    kc_ref, vc_ref = kc.clone(), vc.clone()

    out = torch.empty_like(q)
    slots = torch.empty(w.S, dtype=torch.int64, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            m.paged_decode_step(q, nk, nv, kc, vc, bt, sl, w.scale, out=out, slot_mapping=slots, workspace=ws,
                                stream=s)
    torch.cuda.synchronize()
    replay_and_compare(g, [out, slots], [out_ref, slots_ref], s)
    # the append wrote the same token to the same slot every time
    assert torch.equal(bits(kc), bits(kc_ref)) and torch.equal(bits(vc), bits(vc_ref))


def test_multi_token_step_graph_replays_match_eager():
    w = pi.make_workload(3, S=72, len_lo=16, len_hi=3000, q_lens=4)
    announce(f"graph capture of the multi-token step: S={w.S} rows={w.rows}")
    m = pkv()
    q, bt, sl, qs = dev(w.q), dev(w.block_tables), dev(w.seq_lens), dev(w.q_start)
    nk, nv, kc, vc = dev(w.new_k), dev(w.new_v), dev(w.k_cache), dev(w.v_cache)
    ws = m.alloc_multi_token_step_workspace(q, kc, vc, bt, w.max_q_len)
    out_ref = torch.empty_like(q)
    slots_ref = torch.empty(w.rows, dtype=torch.int64, device="cuda")
    m.paged_multi_token_step(q, nk, nv, kc, vc, qs, w.max_q_len, bt, sl, w.scale, out=out_ref,
                             slot_mapping=slots_ref, workspace=ws)
    torch.cuda.synchronize()
    out = torch.empty_like(q)
    slots = torch.empty(w.rows, dtype=torch.int64, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            m.paged_multi_token_step(q, nk, nv, kc, vc, qs, w.max_q_len, bt, sl, w.scale, out=out,
                                     slot_mapping=slots, workspace=ws, stream=s)
    torch.cuda.synchronize()
    replay_and_compare(g, [out, slots], [out_ref, slots_ref], s)
