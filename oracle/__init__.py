"""CPU oracle for paged decode attention and the KV append (fp64).

TEST INFRASTRUCTURE.  Only `tests/`, `__graft_entry__.smoke()` and the
CPU-baseline leg of `bench.py` may import this package.  It shares no code
with the GPU path and imports nothing from it.

The arithmetic lives in `pkv_oracle.c` (plain C, fp64, optional OpenMP over
(sequence, query head)); this module only marshals numpy arrays.  The
pure-Python `brute` module re-checks it on tiny inputs.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pkv_oracle.c")
_LIB = os.path.join(_HERE, "liborc.so")

ORC_F32 = 0
ORC_BF16 = 1
ORC_FP8 = 2


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (fp64, no fast-math, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-fopenmp",
                               "-fno-fast-math", "-ffp-contract=off", "-shared", "-fPIC",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _bind(path: str):
    L = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i32, i64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    L.orc_key_index.restype = ctypes.c_size_t
    L.orc_key_index.argtypes = [i64, i64, i64, i64, i32, i32, i32, i32]
    L.orc_value_index.restype = ctypes.c_size_t
    L.orc_value_index.argtypes = [i64, i64, i64, i64, i32, i32, i32]
    L.orc_slot_of_position.restype = i64
    L.orc_slot_of_position.argtypes = [P, i64, i32]
    L.orc_slot_split.restype = None
    L.orc_slot_split.argtypes = [i64, i32, P, P]
    L.orc_decode_slot_mapping.restype = None
    L.orc_decode_slot_mapping.argtypes = [P, P, i32, i32, i32, P]
    L.orc_kv_append.restype = None
    L.orc_kv_append.argtypes = [P, P, P, i32, i32, i32, i32, i32, P, P]
    L.orc_paged_attention.restype = ctypes.c_int
    L.orc_paged_attention.argtypes = [P, P, P, P, P, i32, i32, i32, i32, i32, i32, i32, f64, P, ctypes.c_int]
    L.orc_paged_attention_units.restype = ctypes.c_int
    L.orc_paged_attention_units.argtypes = [P, P, P, P, P, i32, i32, i32, i32, i32, i32, i32, f64, P, i64, P,
                                            ctypes.c_int]
    L.orc_paged_attention_split.restype = ctypes.c_int
    L.orc_paged_attention_split.argtypes = [P, P, P, P, P, i32, i32, i32, i32, i32, i32, i32, f64, i32, P,
                                            ctypes.c_int]
    L.orc_max_threads.restype = ctypes.c_int
    L.orc_max_threads.argtypes = []
    L.orc_fp8_decode.restype = f64
    L.orc_fp8_decode.argtypes = [ctypes.c_uint8]
    L.orc_fp8_encode.restype = ctypes.c_uint8
    L.orc_fp8_encode.argtypes = [ctypes.c_float]
    L.orc_fp8_quantize.restype = None
    L.orc_fp8_quantize.argtypes = [P, i64, i32, ctypes.c_float, P]
    L.orc_kv_append_fp8.restype = None
    L.orc_kv_append_fp8.argtypes = [P, P, P, i32, i32, i32, i32, i32, ctypes.c_float, ctypes.c_float, P, P]
    L.orc_multi_token_slot_mapping.restype = None
    L.orc_multi_token_slot_mapping.argtypes = [P, P, P, i32, i32, i32, P]
    L.orc_paged_multi_token_attention.restype = ctypes.c_int
    L.orc_paged_multi_token_attention.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, i32, i32, i32, i32, f64, f64, f64,
                                              P, ctypes.c_int]
    L.orc_paged_attention_units_kv.restype = ctypes.c_int
    L.orc_paged_attention_units_kv.argtypes = [P, P, P, P, P, i32, i32, i32, i32, i32, i32, i32, i32, f64, f64,
                                               f64, P, i64, P, ctypes.c_int]
    return L


_lib = None
_override = None


def lib():
    """The loaded C library (building it first if needed)."""
    global _lib
    if _override is not None:
        return _override
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = _bind(_LIB)
    return _lib


class use_library:
    """Context manager: route this module's calls to another build of the
    oracle source (the mutation tests use it to check that the pins catch
    planted mistakes)."""

    def __init__(self, path: str):
        self.L = _bind(path)

    def __enter__(self):
        global _override
        self._prev = _override
        _override = self.L
        return self

    def __exit__(self, *exc):
        global _override
        _override = self._prev
        return False


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return ORC_F32
    if a.dtype == np.uint16:
        return ORC_BF16
    raise TypeError(f"unsupported element type {a.dtype}")


# ---- layout / slot helpers --------------------------------------------------

def key_index(b, h, t, d, Hkv, B, hs, x) -> int:
    return int(lib().orc_key_index(b, h, t, d, Hkv, B, hs, x))


def value_index(b, h, t, d, Hkv, B, hs) -> int:
    return int(lib().orc_value_index(b, h, t, d, Hkv, B, hs))


def slot_of_position(table_row, pos: int, B: int) -> int:
    row = np.ascontiguousarray(table_row, dtype=np.int32)
    return int(lib().orc_slot_of_position(_ptr(row), pos, B))


def slot_split(slot: int, B: int) -> tuple[int, int]:
    b = ctypes.c_int64()
    o = ctypes.c_int64()
    lib().orc_slot_split(slot, B, ctypes.byref(b), ctypes.byref(o))
    return b.value, o.value


def decode_slot_mapping(block_tables: np.ndarray, seq_lens: np.ndarray, B: int) -> np.ndarray:
    t = np.ascontiguousarray(block_tables, dtype=np.int32)
    L = np.ascontiguousarray(seq_lens, dtype=np.int32)
    S, M = t.shape
    out = np.empty(S, dtype=np.int64)
    lib().orc_decode_slot_mapping(_ptr(t), _ptr(L), S, M, B, _ptr(out))
    return out


def multi_token_slot_mapping(block_tables: np.ndarray, seq_lens: np.ndarray, q_start: np.ndarray,
                             B: int) -> np.ndarray:
    """Slots of the query rows: row i of sequence s at position L_s - n_s + i."""
    t = np.ascontiguousarray(block_tables, dtype=np.int32)
    L = np.ascontiguousarray(seq_lens, dtype=np.int32)
    qs = np.ascontiguousarray(q_start, dtype=np.int32)
    S, M = t.shape
    out = np.empty(int(qs[-1]), dtype=np.int64)
    lib().orc_multi_token_slot_mapping(_ptr(t), _ptr(L), _ptr(qs), S, M, B, _ptr(out))
    return out


def kv_append(k: np.ndarray, v: np.ndarray, slots: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray) -> None:
    """In place: write token i's K/V ([T, Hkv, hs]) into slot slots[i]."""
    T, Hkv, hs = k.shape
    B = v_pool.shape[-1]
    dt = _dtype_code(k_pool)
    assert k.dtype == v.dtype == k_pool.dtype == v_pool.dtype
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    s = np.ascontiguousarray(slots, dtype=np.int64)
    lib().orc_kv_append(_ptr(k), _ptr(v), _ptr(s), T, Hkv, hs, B, dt, _ptr(k_pool), _ptr(v_pool))


# ---- attention --------------------------------------------------------------

def paged_attention(q, k_pool, v_pool, block_tables, seq_lens, scale, *, Hkv=None, threads=0,
                    return_threads=False):
    """fp64 [S, Hq, hs]: softmax(scale * q K^T) V over each sequence's tokens,
    K/V gathered through the block table."""
    q = np.ascontiguousarray(q)
    S, Hq, hs = q.shape
    nb, Hkv_, _, B, _ = k_pool.shape
    t = np.ascontiguousarray(block_tables, dtype=np.int32)
    L = np.ascontiguousarray(seq_lens, dtype=np.int32)
    out = np.empty((S, Hq, hs), dtype=np.float64)
    n = lib().orc_paged_attention(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(t), _ptr(L), S, Hq, Hkv_, hs, B,
                                  t.shape[1], _dtype_code(q), float(scale), _ptr(out), int(threads))
    return (out, n) if return_threads else out


def paged_attention_units(q, k_pool, v_pool, block_tables, seq_lens, scale, units, *, threads=0,
                          return_threads=False):
    """fp64 [len(units), hs]: the attention output of the selected
    (sequence, query head) units, unit = s * Hq + h."""
    q = np.ascontiguousarray(q)
    S, Hq, hs = q.shape
    nb, Hkv_, _, B, _ = k_pool.shape
    t = np.ascontiguousarray(block_tables, dtype=np.int32)
    L = np.ascontiguousarray(seq_lens, dtype=np.int32)
    u = np.ascontiguousarray(units, dtype=np.int64)
    out = np.empty((len(u), hs), dtype=np.float64)
    n = lib().orc_paged_attention_units(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(t), _ptr(L), S, Hq, Hkv_, hs,
                                        B, t.shape[1], _dtype_code(q), float(scale), _ptr(u), len(u), _ptr(out),
                                        int(threads))
    return (out, n) if return_threads else out


def paged_attention_split(q, k_pool, v_pool, block_tables, seq_lens, scale, P, *, threads=0):
    """Same result through P-token context partitions merged by log-sum-exp."""
    q = np.ascontiguousarray(q)
    S, Hq, hs = q.shape
    nb, Hkv_, _, B, _ = k_pool.shape
    t = np.ascontiguousarray(block_tables, dtype=np.int32)
    L = np.ascontiguousarray(seq_lens, dtype=np.int32)
    out = np.empty((S, Hq, hs), dtype=np.float64)
    lib().orc_paged_attention_split(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(t), _ptr(L), S, Hq, Hkv_, hs, B,
                                    t.shape[1], _dtype_code(q), float(scale), int(P), _ptr(out), int(threads))
    return out


def max_threads() -> int:
    return int(lib().orc_max_threads())


def decode_step(w, threads=0, return_threads=False):
    """One decode step on a workload: slot mapping, append into copies of the
    pools, attention.  Returns (slots, k_pool, v_pool, out[fp64])."""
    slots = decode_slot_mapping(w.block_tables, w.seq_lens, w.B)
    kp = w.k_cache.copy()
    vp = w.v_cache.copy()
    if w.dtype == "fp8":
        kv_append_fp8(w.new_k, w.new_v, slots, kp, vp, fp8_inv_scale(w.k_scale), fp8_inv_scale(w.v_scale))
        out = paged_attention_fp8(w.q, kp, vp, w.block_tables, w.seq_lens, w.scale, w.k_scale, w.v_scale,
                                  threads=threads)
        r = (out, max_threads() if threads <= 0 else threads) if return_threads else out
    else:
        kv_append(w.new_k, w.new_v, slots, kp, vp)
        r = paged_attention(w.q, kp, vp, w.block_tables, w.seq_lens, w.scale, threads=threads,
                            return_threads=return_threads)
    if return_threads:
        out, n = r
        return slots, kp, vp, out, n
    return slots, kp, vp, r


# ---- FP8 (E4M3) cache elements ---------------------------------------------
# Reading (the pages fix no format or scale): OCP E4M3 codes, one scale per
# pool; a value x is stored as the code nearest to fp32(x * inv_scale) (ties to
# the even mantissa, magnitudes above 448 saturate) and read as value * scale.

def fp8_inv_scale(scale: float) -> float:
    """The fp32 reciprocal of a pool scale, as the append multiplies by it."""
    return float(np.float32(1.0) / np.float32(scale))


def fp8_decode(code: int) -> float:
    return float(lib().orc_fp8_decode(int(code)))


def fp8_encode(v: float) -> int:
    return int(lib().orc_fp8_encode(float(v)))


def fp8_quantize(x: np.ndarray, inv_scale: float) -> np.ndarray:
    """uint8 codes of fp32 or bf16-bit (uint16) values times inv_scale."""
    x = np.ascontiguousarray(x)
    out = np.empty(x.shape, dtype=np.uint8)
    lib().orc_fp8_quantize(_ptr(x), x.size, _dtype_code(x), float(np.float32(inv_scale)), _ptr(out))
    return out


def kv_append_fp8(k: np.ndarray, v: np.ndarray, slots: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray,
                  k_inv_scale: float, v_inv_scale: float) -> None:
    """In place: quantize token i's K/V ([T, Hkv, hs], fp32 or bf16 bits) into
    slot slots[i] of uint8 pools (key [nb, Hkv, hs/16, B, 16], value
    [nb, Hkv, hs, B])."""
    T, Hkv, hs = k.shape
    B = v_pool.shape[-1]
    assert k_pool.dtype == v_pool.dtype == np.uint8 and k.dtype == v.dtype
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    s = np.ascontiguousarray(slots, dtype=np.int64)
    lib().orc_kv_append_fp8(_ptr(k), _ptr(v), _ptr(s), T, Hkv, hs, B, _dtype_code(k),
                            float(np.float32(k_inv_scale)), float(np.float32(v_inv_scale)), _ptr(k_pool), _ptr(v_pool))


def paged_attention_fp8(q, k_pool, v_pool, block_tables, seq_lens, scale, k_scale, v_scale, *, units=None,
                        threads=0):
    """fp64 attention over uint8 E4M3 pools read as code value * k_scale /
    v_scale; q fp32 or bf16 bits.  Every unit ([S, Hq, hs]) or the listed
    units (rows s * Hq + h)."""
    q = np.ascontiguousarray(q)
    S, Hq, hs = q.shape
    nb, Hkv, _, B, _ = k_pool.shape
    t = np.ascontiguousarray(block_tables, dtype=np.int32)
    L = np.ascontiguousarray(seq_lens, dtype=np.int32)
    if units is None:
        out = np.empty((S, Hq, hs), dtype=np.float64)
        uptr, n = None, 0
    else:
        u = np.ascontiguousarray(units, dtype=np.int64)
        out = np.empty((len(u), hs), dtype=np.float64)
        uptr, n = _ptr(u), len(u)
    lib().orc_paged_attention_units_kv(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(t), _ptr(L), S, Hq, Hkv, hs, B,
                                       t.shape[1], _dtype_code(q), ORC_FP8, float(k_scale), float(v_scale),
                                       float(scale), uptr, n, _ptr(out), int(threads))
    return out


# ---- several query tokens per sequence -------------------------------------

def paged_multi_token_attention(q, q_start, k_pool, v_pool, block_tables, seq_lens, scale, *, k_scale=1.0,
                            v_scale=1.0, threads=0):
    """fp64 [rows, Hq, hs]: query row i of sequence s (rows q_start[s] ..
    q_start[s+1]-1, the last tokens of its seq_lens[s]) attends the positions
    up to its own (causal).  Pools: fp32, bf16 bits or uint8 E4M3 codes."""
    q = np.ascontiguousarray(q)
    rows, Hq, hs = q.shape
    kv_dt = ORC_FP8 if k_pool.dtype == np.uint8 else _dtype_code(k_pool)
    Hkv, B = k_pool.shape[1], k_pool.shape[3]
    t = np.ascontiguousarray(block_tables, dtype=np.int32)
    L = np.ascontiguousarray(seq_lens, dtype=np.int32)
    qs = np.ascontiguousarray(q_start, dtype=np.int32)
    assert qs[-1] == rows and len(qs) == len(L) + 1
    out = np.empty((rows, Hq, hs), dtype=np.float64)
    lib().orc_paged_multi_token_attention(_ptr(q), _ptr(qs), _ptr(k_pool), _ptr(v_pool), _ptr(t), _ptr(L), len(L), Hq,
                                      Hkv, hs, B, t.shape[1], _dtype_code(q), kv_dt, float(k_scale), float(v_scale),
                                      float(scale), _ptr(out), int(threads))
    return out


def multi_token_step(w, threads=0):
    """One step with several query tokens per sequence (w.q_start set): slot
    mapping of the rows, append of all of them into copies of the pools,
    causal attention.  Returns (slots, k_pool, v_pool, out[fp64])."""
    slots = multi_token_slot_mapping(w.block_tables, w.seq_lens, w.q_start, w.B)
    kp = w.k_cache.copy()
    vp = w.v_cache.copy()
    if w.dtype == "fp8":
        kv_append_fp8(w.new_k, w.new_v, slots, kp, vp, fp8_inv_scale(w.k_scale), fp8_inv_scale(w.v_scale))
    else:
        kv_append(w.new_k, w.new_v, slots, kp, vp)
    out = paged_multi_token_attention(w.q, w.q_start, kp, vp, w.block_tables, w.seq_lens, w.scale,
                                      k_scale=w.k_scale, v_scale=w.v_scale, threads=threads)
    return slots, kp, vp, out
