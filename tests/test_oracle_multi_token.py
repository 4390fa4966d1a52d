"""Pins of the oracle's attention with several query tokens per sequence.

The pages name chunked prefill (a long prompt's prefill split into chunks
interleaved with decode: "vLLM 核心工程深度剖析", section 6.1), prefill of
the tokens that missed the prefix cache ("PagedAttention 详解：缓存的存储结构",
"分配与增长") and speculative decoding (the deep-dive page, section 9) as
users of the paged cache; all of them attend with several new tokens per
sequence.  Reading: the n new tokens are the last n of the sequence's L
cached tokens (appended first, as in a decode step) and each attends to
every token up to and including its own position (the causal rule of a
decoder).  The pins check that reading against a library routine's own
causal attention, against a pure-Python brute force, and against closed
forms, never against the oracle itself.
"""
import numpy as np
import pytest
import torch

import oracle
import oracle.brute as brute
import pkv_inputs as pi
from test_oracle_pins import as_f64, contiguous_kv


def test_multi_token_slot_mapping_places_rows_at_the_end():
    # 35 tokens in blocks [7, 3, 12] with B = 16 (the cache-structure page's
    # block-table example): the last 4 tokens are positions 31..34, i.e.
    # block 3 offset 15, then block 12 offsets 0..2
    w = pi.make_workload(1, q_lens=[4, 1, 1, 2])
    slots = oracle.multi_token_slot_mapping(w.block_tables, w.seq_lens, w.q_start, w.B)
    assert list(slots[:4]) == [3 * 16 + 15, 12 * 16 + 0, 12 * 16 + 1, 12 * 16 + 2]
    assert len(slots) == 8


def test_one_query_token_each_equals_a_decode_step():
    w = pi.make_workload(3, S=5, len_lo=16, len_hi=90, q_lens=1)
    d = pi.make_workload(3, S=5, len_lo=16, len_hi=90)
    _, _, _, out = oracle.multi_token_step(w)
    _, _, _, ref = oracle.decode_step(d)
    assert np.array_equal(out, ref)


def _full_causal_reference(w, kp, vp, seed=7):
    """Rows of each sequence from the library's causal attention over the
    whole sequence (every position a query, upper-left aligned mask on an
    L x L problem): the last n rows are the query tokens, the earlier rows
    are filler that the causal rule keeps from influencing them."""
    g = np.random.default_rng(seed)
    qf = as_f64(w.q, w.dtype)
    res = np.zeros((w.rows, w.Hq, w.hs))
    G = w.Hq // w.Hkv
    for s, (K, V) in enumerate(contiguous_kv(w, kp, vp)):
        L = len(K)
        n = int(w.q_start[s + 1] - w.q_start[s])
        if n == 0:
            continue
        Q = g.standard_normal((L, w.Hq, w.hs))
        Q[L - n:] = qf[w.q_start[s]:w.q_start[s + 1]]
        Qt = torch.from_numpy(np.ascontiguousarray(Q.transpose(1, 0, 2)))
        Kt = torch.from_numpy(np.ascontiguousarray(K.transpose(1, 0, 2))).repeat_interleave(G, dim=0)
        Vt = torch.from_numpy(np.ascontiguousarray(V.transpose(1, 0, 2))).repeat_interleave(G, dim=0)
        o = torch.nn.functional.scaled_dot_product_attention(Qt, Kt, Vt, is_causal=True, scale=w.scale)
        res[w.q_start[s]:w.q_start[s + 1]] = o[:, L - n:, :].numpy().transpose(1, 0, 2)
    return res


@pytest.mark.parametrize("cfg,kw", [
    (1, dict(q_lens=[5, 16, 1, 50])),
    (2, dict(S=3, len_lo=30, len_hi=70, q_lens=[7, 1, 30])),
    (3, dict(S=5, len_lo=16, len_hi=90, q_lens=4)),
    (4, dict(S=2, len_lo=40, len_hi=130, q_lens=[33, 9])),
    (5, dict(S=4, len_hi=64, q_lens=1)),
])
def test_matches_library_causal_attention(cfg, kw):
    w = pi.make_workload(cfg, **kw)
    _, kp, vp, out = oracle.multi_token_step(w)
    ref = _full_causal_reference(w, kp, vp)
    assert np.abs(out - ref).max() <= 1e-12


def test_matches_pure_python_brute_force():
    w = pi.make_workload(3, S=3, len_lo=16, len_hi=40, hs=64, Hq=8, Hkv=2, q_lens=[3, 16, 1])
    _, kp, vp, out = oracle.multi_token_step(w)
    bf = brute.causal_attention(w.q.tolist(), [int(v) for v in w.q_start], kp.reshape(-1).tolist(),
                                vp.reshape(-1).tolist(), w.block_tables.tolist(), w.seq_lens.tolist(), w.scale,
                                w.Hq, w.Hkv, w.hs, w.B, True)
    assert np.abs(out - np.array(bf)).max() <= 1e-12


def test_first_row_of_a_full_prefill_returns_the_first_value():
    # n = L: row 0 sits at position 0 and sees only token 0
    w = pi.make_workload(1, q_lens=[35, 16, 1, 50])
    _, kp, vp, out = oracle.multi_token_step(w)
    for s, (K, V) in enumerate(contiguous_kv(w, kp, vp)):
        r0 = int(w.q_start[s])
        for h in range(w.Hq):
            assert np.array_equal(out[r0, h], V[0, h // w.G])


def test_zero_query_averages_the_visible_prefix():
    w = pi.make_workload(1, q_lens=[5, 16, 1, 50])
    w.q[:] = 0
    _, kp, vp, out = oracle.multi_token_step(w)
    for s, (K, V) in enumerate(contiguous_kv(w, kp, vp)):
        L = len(K)
        n = int(w.q_start[s + 1] - w.q_start[s])
        for i in range(n):
            mean = V[:L - n + i + 1].mean(axis=0)
            assert np.abs(out[w.q_start[s] + i] - mean).max() <= 1e-12


def test_later_tokens_do_not_change_earlier_rows():
    # the causal rule: overwriting the keys and values after a row's position
    # (here: the whole chunk after row 2) leaves rows 0..2 bit-identical
    w = pi.make_workload(1, q_lens=[6, 1, 1, 1])
    _, kp, vp, out = oracle.multi_token_step(w)
    slots = oracle.multi_token_slot_mapping(w.block_tables, w.seq_lens, w.q_start, w.B)
    kp2, vp2 = kp.copy(), vp.copy()
    for sl in slots[3:6]:
        b, o = divmod(int(sl), w.B)
        kp2[b, :, :, o, :] = 1e3
        vp2[b, :, :, o] = -1e3
    out2 = oracle.paged_multi_token_attention(w.q, w.q_start, kp2, vp2, w.block_tables, w.seq_lens, w.scale)
    assert np.array_equal(out2[:3], out[:3])
    assert not np.array_equal(out2[3:6], out[3:6])


def test_fp8_pools_match_library_on_decoded_values():
    w = pi.make_workload(3, S=3, len_lo=16, len_hi=60, dtype="fp8", q_lens=[5, 2, 9])
    _, kp, vp, out = oracle.multi_token_step(w)
    # the pools' real values (code * scale, fp64) laid out as a 4-wide key pool,
    # then the library route
    table = np.array([oracle.fp8_decode(c) for c in range(256)])
    kd = (table[kp] * w.k_scale).transpose(0, 1, 3, 2, 4).reshape(w.num_blocks, w.Hkv, w.B, w.hs)
    k4 = np.ascontiguousarray(kd.reshape(w.num_blocks, w.Hkv, w.B, w.hs // 4, 4).transpose(0, 1, 3, 2, 4))
    vd = table[vp] * w.v_scale
    wf = pi.Workload(**{**w.__dict__, "dtype": "f32", "q": pi.f32_from_bf16_bits(w.q)})
    ref = _full_causal_reference(wf, k4, vd)
    assert np.abs(out - ref).max() <= 1e-12
