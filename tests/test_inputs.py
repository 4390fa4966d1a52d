"""The seeded input generators: determinism and the structure of each
configuration (lengths, tables, sharing, poison)."""
import numpy as np
import pytest

import pkv_inputs as pi


def test_bf16_rounding_is_nearest_even():
    a = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, np.inf], dtype=np.float32)
    bits = pi.bf16_bits_from_f32(a)
    back = pi.f32_from_bf16_bits(bits)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> even (1.0); 1 + 3*2^-8 -> 1 + 2^-6
    assert list(back) == [1.0, 1.0, 1.0 + 2 ** -6, 1.0, -2.5, np.inf]


@pytest.mark.parametrize("cfg", [1, 2, 3, 5])
def test_generation_is_deterministic(cfg):
    kw = {} if cfg == 1 else dict(S=4)
    if cfg == 5:
        kw = dict(S=4, len_hi=64)
    a = pi.make_workload(cfg, **kw)
    b = pi.make_workload(cfg, **kw)
    for f in ("seq_lens", "block_tables", "q", "k_cache", "v_cache", "new_k", "new_v"):
        assert getattr(a, f).tobytes() == getattr(b, f).tobytes()


def test_config1_structure():
    w = pi.make_workload(1)
    assert list(w.seq_lens) == [35, 16, 1, 50]
    assert list(w.block_tables[0, :3]) == [7, 3, 12]
    assert w.num_blocks == 32 and w.M == 4 and w.dtype == "f32" and w.hs == 64
    used = set()
    for s in range(w.S):
        n = -(-int(w.seq_lens[s]) // w.B)
        used.update(int(b) for b in w.block_tables[s, :n])
        assert all(int(b) == w.poison_block for b in w.block_tables[s, n:])
    assert w.poison_block not in used and len(used) == 9
    assert np.isnan(w.k_cache[w.poison_block]).all()


def test_config2_lengths_and_pool():
    w = pi.make_workload(2, mode="timing")
    assert w.S == 64 and w.num_blocks == 8192 and w.M == 128
    assert w.seq_lens.min() >= 128 and w.seq_lens.max() <= 2048
    ids = np.concatenate([w.block_tables[s, :-(-int(w.seq_lens[s]) // 16)] for s in range(w.S)])
    assert len(np.unique(ids)) == len(ids)  # no block shared


def test_config3_lengths():
    w = pi.make_workload(3, mode="timing")
    L = w.seq_lens
    assert w.S == 256 and L.min() >= 16 and L.max() <= 8192
    assert 600 < np.median(L) < 1600
    need = sum(-(-int(x) // 16) for x in L)
    assert w.num_blocks >= int(np.ceil(1.1 * need))


def test_config5_sharing():
    w = pi.make_workload(5, mode="timing")
    assert w.S == 128 and (w.seq_lens > 2048).all() and (w.seq_lens <= 2560).all()
    first = w.block_tables[:, :128]
    assert (first == first[0]).all()
    assert (w.ref_count[first[0]] == 128).all()
    tails = np.concatenate([w.block_tables[s, 128:-(-int(w.seq_lens[s]) // 16)] for s in range(w.S)])
    assert len(np.unique(tails)) == len(tails)
    assert not np.isin(tails, first[0]).any()


def test_append_slot_is_empty_before_the_step():
    w = pi.make_workload(2, S=5, len_lo=20, len_hi=100)
    for s in range(w.S):
        pos = int(w.seq_lens[s]) - 1
        b = int(w.block_tables[s, pos // w.B])
        assert np.all(w.k_cache[b, :, :, pos % w.B, :] == pi.BF16_NAN)
