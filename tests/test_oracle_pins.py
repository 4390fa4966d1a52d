"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these compare the oracle with itself: they check it against values
the pages print (tests/golden/, each with its citation), against a library
routine on a contiguous copy of the same K/V, against a pure-Python brute
force on tiny inputs, against closed forms of softmax attention, and against
invariances the pages state (paging changes only where K/V live).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import oracle.brute as brute
import pkv_inputs as pi
from conftest import golden


def as_f64(a, dtype):
    return pi.f32_from_bf16_bits(a).astype(np.float64) if dtype == "bf16" else a.astype(np.float64)


# ---------------------------------------------------------------------------
# worked examples printed on the pages
# ---------------------------------------------------------------------------

def test_block_table_example_token_placement():
    g = golden("block_table_example.json")
    B = g["block_size"]
    row = np.array(g["block_table"], dtype=np.int32)
    for lo, hi, blk in g["token_ranges"]:
        for pos in range(lo, hi + 1):
            b, off = oracle.slot_split(oracle.slot_of_position(row, pos, B), B)
            assert b == blk and off == pos - (pos // B) * B
    # the last block holds exactly 3 tokens: positions 32..34
    last = [p for p in range(g["num_tokens"]) if oracle.slot_split(oracle.slot_of_position(row, p, B), B)[0] == 12]
    assert len(last) == g["last_block_filled"]


def test_slot_mapping_example():
    g = golden("slot_example.json")
    row = np.array(g["block_table"], dtype=np.int32)
    got = [oracle.slot_of_position(row, p, g["block_size"]) for p in g["positions"]]
    assert got == g["slots"]


def test_decode_slot_mapping_uses_last_position():
    # the 35-token request of the block-table example appends position 34 -> slot 194
    g = golden("slot_example.json")
    tables = np.array([g["block_table"], [5, 0, 0]], dtype=np.int32)
    lens = np.array([35, 0], dtype=np.int32)
    assert list(oracle.decode_slot_mapping(tables, lens, 16)) == [194, -1]


def test_key_address_example():
    g = golden("address_example.json")
    B, hs, Hkv, x = g["block_size"], g["head_size"], g["num_kv_heads"], g["x"]
    row = np.array(g["block_table"], dtype=np.int32)
    slot = oracle.slot_of_position(row, g["position"], B)
    blk, off = oracle.slot_split(slot, B)
    assert (g["position"] // B, blk, off) == (g["block_idx"], g["block_number"], g["block_offset"])
    assert oracle.key_index(blk, g["kv_head"], off, 0, Hkv, B, hs, x) == g["key_offset"]
    # strides printed next to the example
    k0 = oracle.key_index(0, 0, 0, 0, Hkv, B, hs, x)
    assert oracle.key_index(1, 0, 0, 0, Hkv, B, hs, x) - k0 == g["kv_block_stride"]
    assert oracle.key_index(0, 1, 0, 0, Hkv, B, hs, x) - k0 == g["kv_head_stride"]
    # x consecutive head dims are contiguous; the next x-chunk is block_size*x further
    assert oracle.key_index(0, 0, 0, 1, Hkv, B, hs, x) - k0 == 1
    assert oracle.key_index(0, 0, 0, x, Hkv, B, hs, x) - k0 == B * x
    assert oracle.key_index(0, 0, 1, 0, Hkv, B, hs, x) - k0 == x


def test_value_address_layout():
    g = golden("address_example.json")
    B, hs, Hkv = g["block_size"], g["head_size"], g["num_kv_heads"]
    v0 = oracle.value_index(0, 0, 0, 0, Hkv, B, hs)
    assert oracle.value_index(1, 0, 0, 0, Hkv, B, hs) - v0 == g["kv_block_stride"]
    assert oracle.value_index(0, 1, 0, 0, Hkv, B, hs) - v0 == g["kv_head_stride"]
    # block_size is the innermost dimension of the value layout
    assert oracle.value_index(0, 0, 1, 0, Hkv, B, hs) - v0 == 1
    assert oracle.value_index(0, 0, 0, 1, Hkv, B, hs) - v0 == B
    # position 20 / head 5 of the example, head dim 7: 3*65536 + 5*2048 + 7*16 + 4
    assert oracle.value_index(3, 5, 4, 7, Hkv, B, hs) == 206964


def test_slot_round_trip_every_slot():
    B, nb = 16, 32
    for slot in range(nb * B):
        b, off = oracle.slot_split(slot, B)
        row = np.array([b], dtype=np.int32)
        assert 0 <= off < B and oracle.slot_of_position(row, off, B) == slot


def test_kv_bytes_formula_reproduces_page_figures():
    g = golden("kv_bytes_examples.json")
    # a one-token, one-layer decode read of d = Hkv * hs elements, keys and values
    w = pi.make_workload(1, S=1, seq_lens=[1])
    per_layer = 1 * g["d_70b"] * 2 * g["bytes_per_elem"]
    assert per_layer * g["layers_70b"] == g["per_token_MiB_70b"] * 2 ** 20
    assert per_layer * g["layers_70b"] * g["tokens_70b"] == g["seq_GiB_70b"] * 2 ** 30
    assert 2 * g["layers_7b"] * g["d_7b"] * g["bytes_per_elem"] == g["per_token_MiB_7b"] * 2 ** 20
    reserved = g["reserve_requests"] * g["reserve_tokens"]
    wasted = reserved - g["reserve_requests"] * g["used_tokens"]
    assert wasted == g["wasted_slots"] and round(100 * wasted / reserved) == g["waste_pct"]
    # the workload's byte count uses the same formula: L * Hkv * hs * 2 * sizeof
    assert w.kv_read_bytes() == 1 * w.Hkv * w.hs * 2 * 4


# ---------------------------------------------------------------------------
# attention arithmetic against independent routes
# ---------------------------------------------------------------------------

def contiguous_kv(w, kp, vp):
    """Per-sequence contiguous K/V [L, Hkv, hs] gathered with numpy axis
    transposes of the pool layouts (no scalar index formula)."""
    x = w.x
    kf = as_f64(kp, w.dtype).reshape(w.num_blocks, w.Hkv, w.hs // x, w.B, x)
    kf = kf.transpose(0, 3, 1, 2, 4).reshape(w.num_blocks, w.B, w.Hkv, w.hs)
    vf = as_f64(vp, w.dtype).reshape(w.num_blocks, w.Hkv, w.hs, w.B).transpose(0, 3, 1, 2)
    out = []
    for s in range(w.S):
        L = int(w.seq_lens[s])
        nblk = -(-L // w.B)
        ids = w.block_tables[s, :nblk]
        K = kf[ids].reshape(nblk * w.B, w.Hkv, w.hs)[:L]
        V = vf[ids].reshape(nblk * w.B, w.Hkv, w.hs)[:L]
        out.append((K, V))
    return out


def sdpa_reference(w, kp, vp):
    qf = as_f64(w.q, w.dtype)
    res = np.zeros((w.S, w.Hq, w.hs))
    for s, (K, V) in enumerate(contiguous_kv(w, kp, vp)):
        if len(K) == 0:
            continue
        G = w.Hq // w.Hkv
        Kt = torch.from_numpy(np.ascontiguousarray(K.transpose(1, 0, 2))).repeat_interleave(G, dim=0)
        Vt = torch.from_numpy(np.ascontiguousarray(V.transpose(1, 0, 2))).repeat_interleave(G, dim=0)
        qt = torch.from_numpy(qf[s]).unsqueeze(1)
        o = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, scale=w.scale)
        res[s] = o[:, 0, :].numpy()
    return res


@pytest.mark.parametrize("cfg,kw", [
    (1, {}),
    (2, dict(S=3, len_lo=30, len_hi=70)),
    (3, dict(S=5, len_lo=16, len_hi=90)),
    (4, dict(S=2, len_lo=40, len_hi=130)),
    (5, dict(S=4, len_hi=64)),
])
def test_oracle_matches_library_sdpa_on_contiguous_copy(cfg, kw):
    w = pi.make_workload(cfg, **kw)
    slots, kp, vp, out = oracle.decode_step(w)
    ref = sdpa_reference(w, kp, vp)
    assert np.abs(out - ref).max() <= 1e-12


def test_oracle_matches_pure_python_brute_force():
    w = pi.make_workload(1)
    slots, kp, vp, out = oracle.decode_step(w)
    bf = brute.attention(w.q.tolist(), kp.reshape(-1).tolist(), vp.reshape(-1).tolist(),
                         w.block_tables.tolist(), w.seq_lens.tolist(), w.scale, w.Hq, w.Hkv, w.hs, w.B, False)
    assert np.abs(out - np.array(bf)).max() <= 1e-12


def test_oracle_matches_brute_force_bf16_gqa():
    w = pi.make_workload(3, S=3, len_lo=16, len_hi=40, hs=64, Hq=8, Hkv=2)
    slots, kp, vp, out = oracle.decode_step(w)
    bf = brute.attention(w.q.tolist(), kp.reshape(-1).tolist(), vp.reshape(-1).tolist(),
                         w.block_tables.tolist(), w.seq_lens.tolist(), w.scale, w.Hq, w.Hkv, w.hs, w.B, True)
    assert np.abs(out - np.array(bf)).max() <= 1e-12


# ---------------------------------------------------------------------------
# closed forms of softmax attention
# ---------------------------------------------------------------------------

def test_single_token_returns_its_value_exactly():
    w = pi.make_workload(1)
    slots, kp, vp, out = oracle.decode_step(w)
    s = int(np.nonzero(w.seq_lens == 1)[0][0])
    for h in range(w.Hq):
        assert np.array_equal(out[s, h], w.new_v[s, h // (w.Hq // w.Hkv)].astype(np.float64))


def test_zero_query_averages_values():
    w = pi.make_workload(1)
    w.q[:] = 0
    slots, kp, vp, out = oracle.decode_step(w)
    for s, (K, V) in enumerate(contiguous_kv(w, kp, vp)):
        mean = V.mean(axis=0)  # [Hkv, hs]
        assert np.abs(out[s] - mean).max() <= 1e-12


def test_dominant_key_selects_its_value():
    w = pi.make_workload(1)
    slots, kp, vp, _ = oracle.decode_step(w)
    s, t = 3, 21  # sequence 3 (50 tokens), logical token 21
    blk, off = int(w.block_tables[s, t // w.B]), t % w.B
    kq = kp.reshape(w.num_blocks, w.Hkv, w.hs // 4, w.B, 4)
    for h in range(w.Hkv):
        kq[blk, h, :, off, :] = (40.0 * w.q[s, h]).reshape(w.hs // 4, 4)
    out = oracle.paged_attention(w.q, kp, vp, w.block_tables, w.seq_lens, w.scale)
    vq = vp.reshape(w.num_blocks, w.Hkv, w.hs, w.B)
    for h in range(w.Hq):
        assert np.abs(out[s, h] - vq[blk, h, :, off]).max() < 1e-9


def test_empty_sequence_gives_zero():
    w = pi.make_workload(1)
    slots, kp, vp, _ = oracle.decode_step(w)
    lens = w.seq_lens.copy()
    lens[1] = 0
    out = oracle.paged_attention(w.q, kp, vp, w.block_tables, lens, w.scale)
    assert np.all(out[1] == 0)
    assert not np.isnan(out[0]).any()


# ---------------------------------------------------------------------------
# invariances the pages state
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("cfg,kw", [(1, {}), (3, dict(S=6, len_lo=16, len_hi=200))])
def test_block_relabelling_leaves_result_bit_identical(cfg, kw):
    w = pi.make_workload(cfg, **kw)
    a = oracle.decode_step(w)
    for seed in (1, 2):
        r = pi.relabel_blocks(w, seed)
        b = oracle.decode_step(r)
        assert np.array_equal(a[3], b[3])


def test_poisoned_unused_slots_do_not_matter():
    wp = pi.make_workload(2, S=4, len_lo=17, len_hi=100, mode="parity")
    wt = pi.make_workload(2, S=4, len_lo=17, len_hi=100, mode="timing")
    assert np.isnan(pi.f32_from_bf16_bits(wp.k_cache)).any()
    assert np.array_equal(oracle.decode_step(wp)[3], oracle.decode_step(wt)[3])


def test_shared_prefix_equals_copied_prefix():
    w = pi.make_workload(5, S=6, len_hi=64)
    assert w.ref_count.max() == 6
    c = pi.unshare_blocks(w)
    assert c.ref_count.max() == 1
    assert np.array_equal(oracle.decode_step(w)[3], oracle.decode_step(c)[3])


def test_sharing_example_tables():
    """The pages' sharing examples as tables over one pool: branches with the
    shared prompt P8 -> P2 -> P15 read the same prefix as a private copy."""
    g = golden("sharing_examples.json")
    nb, Hkv, Hq, hs, B = 32, 2, 4, 64, 16
    scale = 1 / 8
    tables = np.array([g["branch_a"], g["branch_b"]], dtype=np.int32)
    lens = np.array([60, 52], dtype=np.int32)
    rng = np.random.default_rng(0)
    kp = rng.standard_normal((nb, Hkv, hs // 4, B, 4)).astype(np.float32)
    vp = rng.standard_normal((nb, Hkv, hs, B)).astype(np.float32)
    q = rng.standard_normal((2, Hq, hs)).astype(np.float32)
    shared = oracle.paged_attention(q, kp, vp, tables, lens, scale)
    # private copies of the prompt for branch B in blocks 20, 21, 22
    kp2, vp2 = kp.copy(), vp.copy()
    for src, dst in zip(g["shared_prompt"], (20, 21, 22)):
        kp2[dst] = kp[src]
        vp2[dst] = vp[src]
    tables2 = np.array([g["branch_a"], [20, 21, 22, 9]], dtype=np.int32)
    copied = oracle.paged_attention(q, kp2, vp2, tables2, lens, scale)
    assert np.array_equal(shared, copied)
    # the two yololab tables share physical blocks 17 and 4
    ta, tb = g["table_a"], g["table_b"]
    assert ta[:2] == tb[:2] and ta[2] != tb[2]


@pytest.mark.parametrize("P", [16, 48, 512, 100000])
def test_partition_merge_equals_direct(P):
    w = pi.make_workload(3, S=6, len_lo=16, len_hi=900)
    slots, kp, vp, out = oracle.decode_step(w)
    split = oracle.paged_attention_split(w.q, kp, vp, w.block_tables, w.seq_lens, w.scale, P)
    assert np.abs(split - out).max() <= 1e-12


def test_sampled_units_match_full():
    w = pi.make_workload(3, S=5, len_lo=16, len_hi=300)
    slots, kp, vp, out = oracle.decode_step(w)
    units = np.array([0, 7, 33, 5 * w.Hq - 1])
    got = oracle.paged_attention_units(w.q, kp, vp, w.block_tables, w.seq_lens, w.scale, units)
    assert np.array_equal(got, out.reshape(-1, w.hs)[units])


# ---------------------------------------------------------------------------
# append
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("cfg,kw", [(1, {}), (5, dict(S=5, len_hi=32))])
def test_append_writes_slots_bit_exactly_and_nothing_else(cfg, kw):
    w = pi.make_workload(cfg, **kw)
    slots = oracle.decode_slot_mapping(w.block_tables, w.seq_lens, w.B)
    kp, vp = w.k_cache.copy(), w.v_cache.copy()
    oracle.kv_append(w.new_k, w.new_v, slots, kp, vp)
    touched_k = np.zeros(kp.shape, bool)
    touched_v = np.zeros(vp.shape, bool)
    for i, slot in enumerate(slots):
        b, off = int(slot) // w.B, int(slot) % w.B
        # axis views of the documented layouts
        kslot = np.ascontiguousarray(kp[b, :, :, off, :]).reshape(w.Hkv, w.hs)
        vslot = np.ascontiguousarray(vp[b, :, :, off])
        assert kslot.tobytes() == np.ascontiguousarray(w.new_k[i]).tobytes()
        assert vslot.tobytes() == np.ascontiguousarray(w.new_v[i]).tobytes()
        touched_k[b, :, :, off, :] = True
        touched_v[b, :, :, off] = True
    assert kp[~touched_k].tobytes() == w.k_cache[~touched_k].tobytes()
    assert vp[~touched_v].tobytes() == w.v_cache[~touched_v].tobytes()


def test_append_skips_negative_slots():
    w = pi.make_workload(1)
    kp, vp = w.k_cache.copy(), w.v_cache.copy()
    oracle.kv_append(w.new_k, w.new_v, np.full(w.S, -1, np.int64), kp, vp)
    assert kp.tobytes() == w.k_cache.tobytes() and vp.tobytes() == w.v_cache.tobytes()


def test_decode_step_reads_the_appended_token():
    """Before the append the new token's slot holds NaN; afterwards the
    output is finite, so the attention reads exactly the appended slot."""
    w = pi.make_workload(2, S=3, len_lo=20, len_hi=60)
    slots, kp, vp, out = oracle.decode_step(w)
    assert np.isfinite(out).all()
    bad = oracle.paged_attention(w.q, w.k_cache, w.v_cache, w.block_tables, w.seq_lens, w.scale)
    assert np.isnan(bad).all(axis=-1).all()
