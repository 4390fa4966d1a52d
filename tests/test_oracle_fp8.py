"""Pins of the oracle's FP8 (E4M3) cache path.

The pages allow an FP8 cache element but fix no format, scale or rounding;
the reading (OCP E4M3, one scale per pool, nearest code of fp32(x * 1/scale),
ties to the even mantissa, saturation at 448) is pinned here against a
library routine (torch's float8_e4m3fn conversion, within the representable
range), the format's closed forms, fp64 SDPA on the dequantized values, and
the already pinned bf16 attention path."""
import numpy as np
import pytest
import torch

import oracle
import pkv_inputs as pi

F8 = torch.float8_e4m3fn


def torch_decode(codes):
    return torch.from_numpy(np.asarray(codes, dtype=np.uint8)).view(F8).to(torch.float64).numpy()


def torch_encode(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(F8).view(torch.uint8).numpy()


def test_decode_matches_the_library_for_every_code():
    mine = np.array([oracle.fp8_decode(c) for c in range(256)])
    ref = torch_decode(np.arange(256))
    assert np.array_equal(np.isnan(mine), np.isnan(ref)) and np.isnan(mine).sum() == 2
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])


def test_closed_forms():
    assert oracle.fp8_decode(0x38) == 1.0 and oracle.fp8_decode(0x7E) == 448.0
    assert oracle.fp8_decode(0x01) == 2.0 ** -9 and oracle.fp8_decode(0x08) == 2.0 ** -6
    assert oracle.fp8_decode(0x80) == 0.0 and np.signbit(oracle.fp8_decode(0x80))
    # every finite code round-trips
    for c in range(256):
        if c & 0x7F != 0x7F:
            assert oracle.fp8_encode(oracle.fp8_decode(c)) == c


def test_encode_matches_the_library_on_ties_and_grids():
    finite = np.array([oracle.fp8_decode(c) for c in range(0x7F)])       # 0 .. 448
    mids = (finite[:-1] + finite[1:]) / 2                                  # exact ties
    grid = np.concatenate([finite, mids, mids * (1 + 2.0 ** -20), mids * (1 - 2.0 ** -20),
                           np.linspace(0, 464, 20001)])
    x = np.concatenate([grid, -grid]).astype(np.float32)
    mine = np.array([oracle.fp8_encode(v) for v in x], dtype=np.uint8)
    assert np.array_equal(mine, torch_encode(x))


def test_saturation_beyond_the_range():
    # the library turns these into NaN; the reading taken here keeps them finite
    for v, c in [(465.0, 0x7E), (1e6, 0x7E), (-500.0, 0xFE), (float("inf"), 0x7E)]:
        assert oracle.fp8_encode(v) == c
    assert oracle.fp8_encode(float("nan")) == 0x7F


def test_quantize_uses_the_fp32_product():
    rng = np.random.default_rng(3)
    x = pi.bf16_bits_from_f32(rng.standard_normal(4096).astype(np.float32) * 3)
    inv = np.float32(1 / 0.037)
    prod = pi.f32_from_bf16_bits(x) * inv                  # fp32 product
    assert np.array_equal(oracle.fp8_quantize(x, float(inv)), torch_encode(prod))


def fp8_pools(rng, nb, Hkv, hs, B):
    k = rng.integers(0, 256, size=(nb, Hkv, hs // 16, B, 16), dtype=np.uint8)
    v = rng.integers(0, 256, size=(nb, Hkv, hs, B), dtype=np.uint8)
    k[(k & 0x7F) == 0x7F] ^= 0x01            # no NaN codes in used slots
    v[(v & 0x7F) == 0x7F] ^= 0x01
    return k, v


def logical_kv(k, v, table, L, B, kvh, k_scale, v_scale):
    """[L, hs] fp64 K and V of one sequence, by numpy axis transposes."""
    Kb = torch_decode(k).transpose(0, 1, 3, 2, 4).reshape(k.shape[0], k.shape[1], B, -1)   # [nb, Hkv, B, hs]
    Vb = torch_decode(v).transpose(0, 1, 3, 2)                                             # [nb, Hkv, B, hs]
    K = np.concatenate([Kb[b, kvh] for b in table])[:L] * k_scale
    V = np.concatenate([Vb[b, kvh] for b in table])[:L] * v_scale
    return K, V


@pytest.mark.parametrize("B,G", [(16, 1), (16, 4), (32, 8)])
def test_fp8_attention_matches_library_sdpa(B, G):
    rng = np.random.default_rng(B + G)
    S, Hkv, hs, nb = 3, 2, 128, 40
    Hq = G * Hkv
    k, v = fp8_pools(rng, nb, Hkv, hs, B)
    lens = np.array([1, 2 * B + 5, 5 * B], dtype=np.int32)
    M = 5
    tables = np.stack([rng.permutation(nb)[:M] for _ in range(S)]).astype(np.int32)
    q = pi.bf16_bits_from_f32(rng.standard_normal((S, Hq, hs)).astype(np.float32))
    scale, ks, vs = 1 / np.sqrt(hs), 0.043, 0.0121
    got = oracle.paged_attention_fp8(q, k, v, tables, lens, scale, ks, vs)
    for s in range(S):
        for h in range(Hq):
            K, V = logical_kv(k, v, tables[s], lens[s], B, h // G, ks, vs)
            qh = pi.f32_from_bf16_bits(q[s, h]).astype(np.float64)
            o = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(qh)[None, None, None], torch.from_numpy(K)[None, None],
                torch.from_numpy(V)[None, None], scale=scale)[0, 0, 0].numpy()
            assert np.max(np.abs(got[s, h] - o)) < 1e-12


def test_fp8_attention_equals_the_bf16_path_for_power_of_two_scales():
    # code values times 2^-3 are exact in bf16: the same attention through the bf16 pools
    rng = np.random.default_rng(9)
    S, Hkv, Hq, hs, B, nb = 2, 2, 4, 64, 16, 12
    k, v = fp8_pools(rng, nb, Hkv, hs, B)
    lens = np.array([37, 16], dtype=np.int32)
    tables = np.array([[3, 7, 1], [5, 0, 0]], dtype=np.int32)
    q = pi.bf16_bits_from_f32(rng.standard_normal((S, Hq, hs)).astype(np.float32))
    ks = vs = 0.125
    kf = (torch_decode(k) * ks).astype(np.float32)     # [nb, Hkv, hs/16, B, 16]
    vf = (torch_decode(v) * vs).astype(np.float32)
    # the same logical elements in the bf16 layout (x = 8)
    kb = pi.bf16_bits_from_f32(kf.transpose(0, 1, 3, 2, 4).reshape(nb, Hkv, B, hs // 8, 8).transpose(0, 1, 3, 2, 4))
    vb = pi.bf16_bits_from_f32(vf)
    assert np.array_equal(pi.f32_from_bf16_bits(kb).transpose(0, 1, 3, 2, 4).reshape(nb, Hkv, B, hs),
                          kf.transpose(0, 1, 3, 2, 4).reshape(nb, Hkv, B, hs))
    a = oracle.paged_attention_fp8(q, k, v, tables, lens, 0.125, ks, vs)
    b = oracle.paged_attention(q, np.ascontiguousarray(kb), vb, tables, lens, 0.125)
    assert np.array_equal(a, b)


def test_fp8_append_places_codes_of_each_token():
    rng = np.random.default_rng(5)
    T, Hkv, hs, B, nb = 5, 2, 128, 16, 6
    k = pi.bf16_bits_from_f32(rng.standard_normal((T, Hkv, hs)).astype(np.float32))
    v = pi.bf16_bits_from_f32(rng.standard_normal((T, Hkv, hs)).astype(np.float32))
    slots = np.array([3, 17, -1, 40, 95], dtype=np.int64)
    kp = np.full((nb, Hkv, hs // 16, B, 16), 0x7F, np.uint8)
    vp = np.full((nb, Hkv, hs, B), 0x7F, np.uint8)
    ki, vi = np.float32(1 / 0.05), np.float32(1 / 0.02)
    oracle.kv_append_fp8(k, v, slots, kp, vp, float(ki), float(vi))
    Kb = kp.transpose(0, 1, 3, 2, 4).reshape(nb, Hkv, B, hs)
    Vb = vp.transpose(0, 1, 3, 2)
    written = set()
    for i, sl in enumerate(slots):
        if sl < 0:
            continue
        b, off = divmod(int(sl), B)
        written.add((b, off))
        assert np.array_equal(Kb[b, :, off], torch_encode(pi.f32_from_bf16_bits(k[i]) * ki))
        assert np.array_equal(Vb[b, :, off], torch_encode(pi.f32_from_bf16_bits(v[i]) * vi))
    for b in range(nb):
        for off in range(B):
            if (b, off) not in written:
                assert np.all(Kb[b, :, off] == 0x7F) and np.all(Vb[b, :, off] == 0x7F)
