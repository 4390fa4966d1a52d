"""Pure-Python brute force for tiny paged-attention inputs (no numpy math).

TEST INFRASTRUCTURE: used only by the tests, to check the C oracle on tiny
inputs with an independent implementation (scalar loops, math.exp).

Follows the definition on the "vLLM engineering deep-dive" page, section 3.1:
look up the physical block of each logical token through the block table,
score it against the query, softmax the scores, weight the values.  The
element positions follow the "cache structure" page's key layout
[blocks][heads][hs/x][B][x] and value layout [blocks][heads][hs][B].
"""
from __future__ import annotations

import math
import struct


def _as_float(bits_or_value, is_bf16: bool) -> float:
    if is_bf16:
        return struct.unpack("<f", struct.pack("<I", int(bits_or_value) << 16))[0]
    return float(bits_or_value)


def attention(q, k_flat, v_flat, tables, lens, scale, Hq, Hkv, hs, B, is_bf16):
    """q: nested list [S][Hq][hs]; k_flat/v_flat: flat lists of pool elements;
    tables: nested list [S][M]; returns nested list [S][Hq][hs] of floats."""
    x = 8 if is_bf16 else 4
    G = Hq // Hkv
    out = []
    for s in range(len(lens)):
        L = int(lens[s])
        rows = []
        for h in range(Hq):
            kvh = h // G
            if L == 0:
                rows.append([0.0] * hs)
                continue
            scores = []
            places = []
            for t in range(L):
                blk = int(tables[s][t // B])
                j = t % B
                places.append((blk, j))
                acc = 0.0
                for d in range(hs):
                    kpos = (((blk * Hkv + kvh) * (hs // x) + d // x) * B + j) * x + d % x
                    acc += _as_float(q[s][h][d], is_bf16) * _as_float(k_flat[kpos], is_bf16)
                scores.append(acc * scale)
            m = max(scores)
            w = [math.exp(sc - m) for sc in scores]
            z = sum(w)
            o = []
            for d in range(hs):
                acc = 0.0
                for (blk, j), wt in zip(places, w):
                    vpos = ((blk * Hkv + kvh) * hs + d) * B + j
                    acc += wt * _as_float(v_flat[vpos], is_bf16)
                o.append(acc / z)
            rows.append(o)
        out.append(rows)
    return out


def causal_attention(q, q_start, k_flat, v_flat, tables, lens, scale, Hq, Hkv, hs, B, is_bf16):
    """Several query rows per sequence with the causal rule: rows q_start[s]
    .. q_start[s+1]-1 of q (nested list [rows][Hq][hs]) are the last n of the
    sequence's L tokens, row i at position L - n + i, and each sees the
    tokens at positions 0 .. its own.  Returns nested list [rows][Hq][hs]."""
    x = 8 if is_bf16 else 4
    G = Hq // Hkv
    out = [None] * q_start[-1]
    for s in range(len(lens)):
        L = int(lens[s])
        n = q_start[s + 1] - q_start[s]
        for i in range(n):
            row = q_start[s] + i
            visible = L - n + i + 1
            heads = []
            for h in range(Hq):
                kvh = h // G
                scores = []
                for t in range(visible):
                    blk = int(tables[s][t // B])
                    j = t % B
                    acc = 0.0
                    for d in range(hs):
                        kpos = (((blk * Hkv + kvh) * (hs // x) + d // x) * B + j) * x + d % x
                        acc += _as_float(q[row][h][d], is_bf16) * _as_float(k_flat[kpos], is_bf16)
                    scores.append(acc * scale)
                m = max(scores)
                w = [math.exp(sc - m) for sc in scores]
                z = sum(w)
                o = []
                for d in range(hs):
                    acc = 0.0
                    for t in range(visible):
                        blk = int(tables[s][t // B])
                        vpos = ((blk * Hkv + kvh) * hs + d) * B + t % B
                        acc += w[t] * _as_float(v_flat[vpos], is_bf16)
                    o.append(acc / z)
                heads.append(o)
            out[row] = heads
    return out
