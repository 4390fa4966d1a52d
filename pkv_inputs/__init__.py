"""Seeded synthetic decode-step inputs for paged attention.

This module is shared by the CPU oracle's tests and by the GPU path's tests
and benchmark.  It holds no part of the attention or append arithmetic: it
draws random numbers, plays the role of the host block allocator (which
physical block IDs each sequence owns and how many slots of each block are
filled), and lays the draws out in the pool formats that the C ABI documents.

Workloads (one per decode configuration):

  1  tiny fp32 decode: 4 sequences, lengths [35, 16, 1, 50], B=16, 8/8 heads,
     head size 64, a pool of 32 blocks; sequence 0 owns blocks [7, 3, 12]
     (the 35-token, B=16 worked example of the "cache structure" page,
     section "Block Table").
  2  MHA bf16 decode: 64 sequences, 32/32 heads, head size 128, B=16, lengths
     uniform on [128, 2048], a pool of 8192 blocks with shuffled IDs.
  3  GQA bf16 decode: 256 sequences, 32/8 heads, head size 128, B=16, lengths
     log-normal (median 1000, sigma 0.8) clipped to [16, 8192], a pool of
     1.1x the needed blocks with shuffled IDs.
  4  long-context bf16 decode: 8 sequences, 64/8 heads, head size 128, B=32,
     lengths uniform on [32768, 131072], values 0.5*N(0,1), 512-token
     context partitions.
  5  shared-prefix fork bf16 decode: 128 branches share one 2048-token prompt
     (128 physical blocks, each referenced by all 128 tables) plus private
     tails of 1..512 tokens; 32/8 heads, head size 128, B=16.

Every decode step appends one token per sequence at position L-1 and then
attends over all L tokens.  With `q_lens` (several query tokens per sequence:
a prefill chunk, or the draft tokens of speculative decoding) sequence s has
n_s = q_lens[s] query tokens, the last n_s of its L_s, stored as rows
q_start[s] .. q_start[s+1]-1 of q and of the new k/v; the step appends all of
them and then attends causally.  Before the append the slot of that position holds
NaN (parity mode), so a missing or misplaced append shows up in the output.

Pool formats (element type T, x = 16 / sizeof(T) elements per 16-byte chunk):
  key pool   [num_blocks, Hkv, hs/x, B, x]
  value pool [num_blocks, Hkv, hs,   B]
bf16 data is carried as uint16 bit patterns produced from float32 draws by
round-to-nearest-even.

Random streams: every array is drawn from numpy PCG64 generators seeded by
SeedSequence(seed, spawn_key=(stream, chunk)); the stream order is
seq_lens (0), block-ID permutation (1), q (2), key pool (3), value pool (4),
new k/v (5).  Large arrays are drawn in fixed 4 Mi-element chunks on a
thread pool, so the values do not depend on the thread count.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

CHUNK = 1 << 22

STREAM_LENS, STREAM_PERM, STREAM_Q, STREAM_K, STREAM_V, STREAM_NEW = range(6)


# ----------------------------------------------------------------------------
# bit-level helpers (format conversion only)
# ----------------------------------------------------------------------------

def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even.

    NaN inputs map to a quiet NaN pattern."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = a.view(np.uint32)
    r = ((b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        r[nan] = np.uint16(0x7FC0)
    return r


def f32_from_bf16_bits(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float32 (exact)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


BF16_NAN = np.uint16(0x7FC0)

# FP8 pools: E4M3 codes (0x7F is a NaN code); per-pool scales, as multiples of
# the draws' standard deviation, chosen so that the largest draws stay well
# inside the format's range (|x / scale| < 448 up to ~10 sigma)
FP8_NAN = np.uint8(0x7F)
FP8_SCALES = (0.0271, 0.0193)


def _fp8_codes(a: np.ndarray, scale: float) -> np.ndarray:
    """E4M3 codes of a / scale through torch's float8_e4m3fn cast (chunked)."""
    import torch

    flat = a.reshape(-1)
    out = np.empty(flat.size, dtype=np.uint8)
    inv = np.float32(1.0 / scale)
    for lo in range(0, flat.size, CHUNK):
        hi = min(flat.size, lo + CHUNK)
        t = torch.from_numpy(flat[lo:hi] * inv)
        out[lo:hi] = t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return out.reshape(a.shape)


def _rng(seed: int, stream: int, chunk: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(stream, chunk))))


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def fill_normal(out: np.ndarray, seed: int, stream: int, std: float = 1.0) -> None:
    """Fill a contiguous array (float32 or uint16 bf16 bits) with std*N(0,1)."""
    flat = out.reshape(-1)
    n = flat.size
    nchunks = (n + CHUNK - 1) // CHUNK

    def work(i: int) -> None:
        lo = i * CHUNK
        hi = min(n, lo + CHUNK)
        a = _rng(seed, stream, i).standard_normal(hi - lo, dtype=np.float32)
        if std != 1.0:
            a *= np.float32(std)
        if flat.dtype == np.uint16:
            flat[lo:hi] = bf16_bits_from_f32(a)
        else:
            flat[lo:hi] = a

    if nchunks <= 1:
        for i in range(nchunks):
            work(i)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nchunks)))


# ----------------------------------------------------------------------------
# host block allocator fixture
# ----------------------------------------------------------------------------

class BlockPoolFixture:
    """Minimal host block allocator used to build decode inputs.

    It hands out physical block IDs in a given order, keeps per-block
    reference counts and per-block fill counts (how many token slots of the
    block already hold data), and records one block table per sequence.
    Modelled on the allocator of the "vLLM engineering deep-dive" page,
    section 2.2 (free list, ref counts, per-request block lists)."""

    def __init__(self, order: np.ndarray, block_size: int):
        self.free = [int(b) for b in order]
        self.free.reverse()  # pop() hands out IDs in `order`
        self.B = block_size
        n = len(order)
        self.ref_count = np.zeros(n, dtype=np.int32)
        self.fill = np.zeros(n, dtype=np.int32)
        self.tables: list[list[int]] = []

    def take(self, count: int) -> list[int]:
        if count > len(self.free):
            raise MemoryError("block pool exhausted")
        ids = [self.free.pop() for _ in range(count)]
        for b in ids:
            self.ref_count[b] += 1
        return ids

    def add_sequence(self, blocks: list[int]) -> None:
        self.tables.append(list(blocks))

    def share(self, blocks: list[int]) -> None:
        for b in blocks:
            self.ref_count[b] += 1

    def write_tokens(self, seq: int, count: int) -> None:
        """Mark `count` more tokens of sequence `seq` as stored: fills the
        sequence's blocks front to back (each block holds B slots)."""
        for b in self.tables[seq]:
            if count <= 0:
                break
            room = self.B - int(self.fill[b])
            if room <= 0:
                continue
            n = min(room, count)
            self.fill[b] += n
            count -= n
        if count > 0:
            raise MemoryError("sequence has no room for more tokens")


# ----------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------

@dataclass
class Workload:
    config: int
    seed: int
    mode: str
    dtype: str                 # "f32" | "bf16" | "fp8" (E4M3 pool codes; q, new k/v in bf16)
    S: int
    Hq: int
    Hkv: int
    hs: int
    B: int
    num_blocks: int
    M: int                     # max_blocks_per_seq (table width)
    scale: float
    partition_tokens: int      # 0 = implementation's choice
    seq_lens: np.ndarray       # int32 [S]
    block_tables: np.ndarray   # int32 [S, M]
    q: np.ndarray              # [rows, Hq, hs] float32 or uint16 bits (rows = S for decode)
    k_cache: np.ndarray        # [nb, Hkv, hs/x, B, x]
    v_cache: np.ndarray        # [nb, Hkv, hs, B]
    new_k: np.ndarray          # [rows, Hkv, hs]
    new_v: np.ndarray          # [rows, Hkv, hs]
    ref_count: np.ndarray      # int32 [nb]
    fill: np.ndarray           # int32 [nb] slots holding data before the append
    poison_block: int
    description: str = ""
    extra: dict = field(default_factory=dict)
    k_scale: float = 1.0       # fp8 pools: stored value = code * scale
    v_scale: float = 1.0
    q_start: Optional[np.ndarray] = None  # int32 [S+1]: query rows of each sequence (None: one each)

    @property
    def rows(self) -> int:
        return self.S if self.q_start is None else int(self.q_start[-1])

    @property
    def max_q_len(self) -> int:
        return 1 if self.q_start is None else int(np.diff(self.q_start).max(initial=0))

    @property
    def x(self) -> int:
        return 16 // self.elem_bytes

    @property
    def elem_bytes(self) -> int:
        return {"f32": 4, "bf16": 2, "fp8": 1}[self.dtype]

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    def kv_read_bytes(self) -> int:
        """Algorithmic KV bytes one decode step reads: every cached token of
        every sequence, once per KV head, keys and values."""
        return int(self.seq_lens.astype(np.int64).sum()) * self.Hkv * self.hs * 2 * self.elem_bytes

    def unique_kv_bytes(self) -> int:
        """Bytes of distinct (block, slot) pairs read: shared blocks count once."""
        seen = {}
        for s in range(self.S):
            L = int(self.seq_lens[s])
            nblk = -(-L // self.B)
            for j in range(nblk):
                b = int(self.block_tables[s, j])
                used = min(self.B, L - j * self.B)
                seen[b] = max(seen.get(b, 0), used)
        return sum(seen.values()) * self.Hkv * self.hs * 2 * self.elem_bytes


_CFG = {
    1: dict(dtype="f32", S=4, Hq=8, Hkv=8, hs=64, B=16, std=1.0,
            desc="tiny paged decode, fp32, seq_lens [35,16,1,50], pool 32 blocks"),
    2: dict(dtype="bf16", S=64, Hq=32, Hkv=32, hs=128, B=16, std=1.0,
            desc="MHA decode layer, bf16, 64 seqs, 32/32 heads, hs 128, B 16, L~U[128,2048], pool 8192 blocks"),
    3: dict(dtype="bf16", S=256, Hq=32, Hkv=8, hs=128, B=16, std=1.0,
            desc="GQA decode layer, bf16, 256 seqs, 32/8 heads, hs 128, B 16, L log-normal(1000,0.8) in [16,8192]"),
    4: dict(dtype="bf16", S=8, Hq=64, Hkv=8, hs=128, B=32, std=0.5,
            desc="long-context split-K decode, bf16, 8 seqs, 64/8 heads, hs 128, B 32, L~U[32768,131072], P=512"),
    5: dict(dtype="bf16", S=128, Hq=32, Hkv=8, hs=128, B=16, std=1.0,
            desc="shared-prefix fork decode, bf16, 128 branches, 2048-token shared prompt + U[1,512] tails"),
}


def config_description(config: int) -> str:
    return _CFG[config]["desc"]


def _draw_lens(config: int, seed: int, S: int, lo: Optional[int], hi: Optional[int]) -> np.ndarray:
    g = _rng(seed, STREAM_LENS)
    if config == 1:
        return np.array([35, 16, 1, 50], dtype=np.int64)[:S]
    if config == 2:
        return g.integers(lo or 128, hi or 2048, size=S, endpoint=True)
    if config == 3:
        z = g.normal(math.log(1000.0), 0.8, size=S)
        return np.clip(np.rint(np.exp(z)), lo or 16, hi or 8192).astype(np.int64)
    if config == 4:
        return g.integers(lo or 32768, hi or 131072, size=S, endpoint=True)
    if config == 5:
        return (hi or 2048) + g.integers(1, 512, size=S, endpoint=True)
    raise ValueError(f"unknown config {config}")


def make_workload(config: int, mode: str = "parity", *, S: Optional[int] = None,
                  len_lo: Optional[int] = None, len_hi: Optional[int] = None,
                  seed: Optional[int] = None, seq_lens: Optional[list] = None,
                  dtype: Optional[str] = None, hs: Optional[int] = None,
                  B: Optional[int] = None, Hq: Optional[int] = None,
                  Hkv: Optional[int] = None, contiguous: bool = False, q_lens=None) -> Workload:
    """Build one decode step's inputs.

    mode "parity": slots and blocks that hold no data are NaN (they must never
    influence a result); mode "timing": they are zero.
    The keyword overrides shrink or reshape a configuration for fast tests
    while keeping its structure (for config 5, `len_hi` is the shared prompt
    length and must be a multiple of B).  q_lens (an int for every sequence,
    or one per sequence; each at most the sequence's length, and for config 5
    within its private tail) gives several query tokens per sequence."""
    if mode not in ("parity", "timing"):
        raise ValueError(mode)
    c = dict(_CFG[config])
    if dtype is not None:
        c["dtype"] = dtype
    for key, val in (("hs", hs), ("B", B), ("Hq", Hq), ("Hkv", Hkv)):
        if val is not None:
            c[key] = val
    seed = config if seed is None else seed
    S = c["S"] if S is None else S
    Bsz = c["B"]
    if seq_lens is not None:
        lens = np.asarray(seq_lens, dtype=np.int64)
        S = len(lens)
    else:
        lens = _draw_lens(config, seed, S, len_lo, len_hi)
    nblk = [-(-int(L) // Bsz) for L in lens]
    M = max(1, max(nblk) if len(nblk) else 1)
    if q_lens is None:
        qn = np.ones(S, dtype=np.int64)
    else:
        qn = np.broadcast_to(np.asarray(q_lens, dtype=np.int64), (S,)).copy()
        if (qn < 0).any() or (qn > lens).any():
            raise ValueError("query tokens must be between 0 and the sequence length")
    rows = int(qn.sum())

    # ---- physical block assignment (allocator fixture) ----
    pg = _rng(seed, STREAM_PERM)
    if contiguous:
        nb_c = {2: 8192}.get(config, 0) if (S == _CFG[config]["S"] and len_hi is None and seq_lens is None) else 0
        need = sum(nblk) if config != 5 else None
        if config == 5:
            prompt = len_hi or 2048
            shared_n = prompt // Bsz
            tails = [n - shared_n for n in nblk]
            need = shared_n + sum(tails)
        nb = max(nb_c, need if config != 3 else int(math.ceil(1.1 * need)))
        order = np.arange(nb)
    elif config == 1 and seq_lens is None and S == 4:
        nb = 32
        rest = np.array([b for b in range(nb) if b not in (7, 3, 12)], dtype=np.int64)
        rest = pg.permutation(rest)
        order = np.concatenate([np.array([7, 3, 12]), rest])
        need = sum(nblk)
    elif config == 5 and not contiguous:
        prompt = len_hi or 2048
        if prompt % Bsz:
            raise ValueError("shared prompt must fill whole blocks")
        shared_n = prompt // Bsz
        tails = [n - shared_n for n in nblk]
        need = shared_n + sum(tails)
        nb = need
        order = pg.permutation(nb)
    else:
        need = sum(nblk)
        if config == 2 and S == _CFG[2]["S"] and len_hi is None:
            nb = 8192
        elif config == 3:
            nb = int(math.ceil(1.1 * need))
        else:
            nb = need
        order = pg.permutation(nb)
    if need < nb:
        poison = int(order[need])
    else:
        poison = nb
        nb += 1
        order = np.concatenate([order, np.array([poison])])
    pool = BlockPoolFixture(order, Bsz)
    if config == 5:
        shared = pool.take(shared_n)
        pool.ref_count[shared] -= 1  # take() counted one owner; add all branches below
        for s in range(S):
            pool.share(shared)
            pool.add_sequence(shared + pool.take(tails[s]))
        pool.write_tokens(0, shared_n * Bsz)  # the prompt is stored once
        for s in range(S):
            # the shared blocks are full, so these tokens land in the tail
            if int(lens[s]) - int(qn[s]) < shared_n * Bsz:
                raise ValueError("query tokens must lie in the private tail")
            pool.write_tokens(s, int(lens[s]) - int(qn[s]) - shared_n * Bsz)
    else:
        for s in range(S):
            pool.add_sequence(pool.take(nblk[s]))
            pool.write_tokens(s, int(lens[s]) - int(qn[s]))
    tables = np.full((S, M), poison, dtype=np.int32)
    for s, row in enumerate(pool.tables):
        tables[s, :len(row)] = row

    # ---- values ----
    dt = c["dtype"]
    Hq_, Hkv_, hs_ = c["Hq"], c["Hkv"], c["hs"]
    if Hq_ % Hkv_:
        raise ValueError("Hq must be a multiple of Hkv")
    esz = {"f32": 4, "bf16": 2, "fp8": 1}[dt]
    x = 16 // esz
    np_t = np.float32 if dt == "f32" else np.uint16   # q and the new k, v (bf16 for fp8 pools)
    std = c["std"]
    q = np.empty((rows, Hq_, hs_), dtype=np_t)
    fill_normal(q, seed, STREAM_Q, std)
    k_scale = v_scale = 1.0
    if dt == "fp8":
        # pool contents as E4M3 codes of the same normal draws divided by a per-pool
        # scale (torch's float8 cast: stored data, not this method's append)
        k_scale, v_scale = FP8_SCALES[0] * std, FP8_SCALES[1] * std
        kf = np.empty((nb, Hkv_, hs_ // x, Bsz, x), dtype=np.float32)
        fill_normal(kf, seed, STREAM_K, std)
        kc = _fp8_codes(kf, k_scale)
        del kf
        vf = np.empty((nb, Hkv_, hs_, Bsz), dtype=np.float32)
        fill_normal(vf, seed, STREAM_V, std)
        vc = _fp8_codes(vf, v_scale)
        del vf
    else:
        kc = np.empty((nb, Hkv_, hs_ // x, Bsz, x), dtype=np_t)
        fill_normal(kc, seed, STREAM_K, std)
        vc = np.empty((nb, Hkv_, hs_, Bsz), dtype=np_t)
        fill_normal(vc, seed, STREAM_V, std)
    new = np.empty((2, rows, Hkv_, hs_), dtype=np_t)
    fill_normal(new, seed, STREAM_NEW, std)

    # slots that hold no data: NaN (parity) or zero (timing)
    if mode == "parity":
        bad = {"f32": np.float32(np.nan), "bf16": BF16_NAN, "fp8": FP8_NAN}[dt]
    else:
        bad = kc.dtype.type(0)
    for b in range(nb):
        f = int(pool.fill[b])
        if f < Bsz:
            kc[b, :, :, f:, :] = bad
            vc[b, :, :, f:] = bad

    scale = 1.0 / math.sqrt(hs_)
    return Workload(config=config, seed=seed, mode=mode, dtype=dt, S=S, Hq=Hq_, Hkv=Hkv_,
                    k_scale=k_scale, v_scale=v_scale,
                    hs=hs_, B=Bsz, num_blocks=nb, M=M, scale=scale,
                    partition_tokens=512 if config == 4 else 0,
                    seq_lens=lens.astype(np.int32), block_tables=tables, q=q,
                    k_cache=kc, v_cache=vc, new_k=new[0], new_v=new[1],
                    ref_count=pool.ref_count.copy(), fill=pool.fill.copy(),
                    poison_block=poison, description=c["desc"],
                    q_start=None if q_lens is None else np.concatenate([[0], np.cumsum(qn)]).astype(np.int32))


def relabel_blocks(w: Workload, seed: int) -> Workload:
    """The same logical content with physical block IDs relabelled by a random
    permutation: block b moves to pi[b] (whole-block moves only)."""
    g = _rng(seed, 99)
    pi = g.permutation(w.num_blocks)
    kc = np.empty_like(w.k_cache)
    vc = np.empty_like(w.v_cache)
    kc[pi] = w.k_cache
    vc[pi] = w.v_cache
    rc = np.empty_like(w.ref_count)
    rc[pi] = w.ref_count
    fl = np.empty_like(w.fill)
    fl[pi] = w.fill
    tables = pi[w.block_tables].astype(np.int32)
    return Workload(**{**w.__dict__, "k_cache": kc, "v_cache": vc, "block_tables": tables,
                       "ref_count": rc, "fill": fl, "poison_block": int(pi[w.poison_block])})


def unshare_blocks(w: Workload) -> Workload:
    """Give every table its own copy of each block that several tables
    reference (whole-block copies appended to the pool)."""
    counts = {}
    for s in range(w.S):
        nblk = -(-int(w.seq_lens[s]) // w.B)
        for j in range(nblk):
            b = int(w.block_tables[s, j])
            counts[b] = counts.get(b, 0) + 1
    shared = sorted(b for b, n in counts.items() if n > 1)
    extra = sum(counts[b] - 1 for b in shared)
    nb = w.num_blocks + extra
    kc = np.concatenate([w.k_cache, np.empty((extra,) + w.k_cache.shape[1:], w.k_cache.dtype)])
    vc = np.concatenate([w.v_cache, np.empty((extra,) + w.v_cache.shape[1:], w.v_cache.dtype)])
    tables = w.block_tables.copy()
    nxt = w.num_blocks
    first = {b: True for b in shared}
    for s in range(w.S):
        nblk = -(-int(w.seq_lens[s]) // w.B)
        for j in range(nblk):
            b = int(tables[s, j])
            if b in first:
                if first[b]:
                    first[b] = False
                    continue
                kc[nxt] = w.k_cache[b]
                vc[nxt] = w.v_cache[b]
                tables[s, j] = nxt
                nxt += 1
    rc = np.ones(nb, dtype=np.int32)
    fl = np.concatenate([w.fill, np.full(extra, w.B, np.int32)])
    return Workload(**{**w.__dict__, "k_cache": kc, "v_cache": vc, "block_tables": tables,
                       "num_blocks": nb, "ref_count": rc, "fill": fl})
