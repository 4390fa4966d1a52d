"""Paged KV-cache decode attention for AMD MI355X (gfx950).

Thin Python binding over the C ABI of libpkv.so (include/pkv.h): it checks
tensor shapes, dtypes and devices, turns tensors into device pointers and
passes torch's current HIP stream.  Every step of the decode path runs in
the library's HIP kernels; there is no Python or CPU fallback, and using the
binding without the built library raises.

Pool layouts (x = 16 / element size):
    k_cache [num_blocks, Hkv, head_size // x, block_size, x]
    v_cache [num_blocks, Hkv, head_size, block_size]
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpkv.so")

PKV_OK = 0
PKV_ERR_OUT_OF_BLOCKS = -5
PKV_F32 = 0
PKV_BF16 = 1
PKV_FP8_E4M3 = 2

# pool element types; FP8 pools hold E4M3 codes (uint8 or float8_e4m3fn tensors)
_DTYPES = {torch.float32: PKV_F32, torch.bfloat16: PKV_BF16, torch.uint8: PKV_FP8_E4M3}
if hasattr(torch, "float8_e4m3fn"):
    _DTYPES[torch.float8_e4m3fn] = PKV_FP8_E4M3


class PkvError(RuntimeError):
    def __init__(self, func: str, status: int, lib):
        name = lib.pkv_status_string(status).decode()
        extra = ""
        if name == "PKV_ERR_HIP":
            extra = " (" + lib.pkv_last_hip_error().decode() + ")"
        super().__init__(f"{func} failed: {name}{extra}")
        self.status = status


class CacheDesc(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("head_size", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float), ("out_f32", ctypes.c_int32)]


_lib = None


def library():
    """The loaded libpkv.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first (python -m paged_kv_cache_35_amd.build "
                               "or __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
        L.pkv_layout_version.restype = i32
        L.pkv_layout_version.argtypes = []
        L.pkv_status_string.restype = ctypes.c_char_p
        L.pkv_status_string.argtypes = [i32]
        L.pkv_last_hip_error.restype = ctypes.c_char_p
        L.pkv_last_hip_error.argtypes = []
        L.pkv_decode_slot_mapping.restype = i32
        L.pkv_decode_slot_mapping.argtypes = [P, P, i32, i32, i32, P, P]
        L.kv_cache_append.restype = i32
        L.kv_cache_append.argtypes = [P, P, P, i32, ctypes.POINTER(CacheDesc), P, P, P]
        L.pkv_decode_append.restype = i32
        L.pkv_decode_append.argtypes = [P, P, P, P, i32, i32, ctypes.POINTER(CacheDesc), P, P, P, P, sz, P]
        L.pkv_decode_schedule_bytes.restype = sz
        L.pkv_decode_schedule_bytes.argtypes = [i32, i32]
        L.pkv_decode_step_workspace_bytes.restype = sz
        L.pkv_decode_step_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32]
        L.pkv_decode_partition_tokens.restype = i32
        L.pkv_decode_partition_tokens.argtypes = [i32, i32, i32, i32, i32, i32, i32]
        L.pkv_decode_workspace_bytes.restype = sz
        L.pkv_decode_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32]
        L.paged_decode_attention.restype = i32
        L.paged_decode_attention.argtypes = [P, P, P, P, P, i32, i32, i32, ctypes.POINTER(CacheDesc), f32, P, P, sz,
                                             i32, P, sz, P]
        L.paged_decode_step.restype = i32
        L.paged_decode_step.argtypes = [P, P, P, P, P, P, P, i32, i32, i32, ctypes.POINTER(CacheDesc), f32, P, P, P,
                                        sz, i32, P]
        L.paged_decode_step_static.restype = i32
        L.paged_decode_step_static.argtypes = [P, P, P, P, P, P, P, i32, i32, i32, ctypes.POINTER(CacheDesc), f32, P,
                                               P, i32, P]
        L.pkv_copy_blocks.restype = i32
        L.pkv_multi_token_workspace_bytes.restype = sz
        L.pkv_multi_token_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32]
        L.pkv_multi_token_slot_mapping.restype = i32
        L.pkv_multi_token_step_workspace_bytes.restype = sz
        L.pkv_multi_token_step_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32]
        L.pkv_multi_token_slot_mapping.argtypes = [P, P, P, i32, i32, i32, i32, i32, P, P, sz, P]
        L.pkv_multi_token_append.restype = i32
        L.pkv_multi_token_append.argtypes = [P, P, P, i32, i32, P, P, i32, i32, ctypes.POINTER(CacheDesc), P, P, P]
        L.paged_multi_token_attention.restype = i32
        L.paged_multi_token_attention.argtypes = [P, P, i32, i32, P, P, P, P, i32, i32, i32,
                                                  ctypes.POINTER(CacheDesc), f32, P, P, sz, i32, P, sz, P]
        L.paged_multi_token_step.restype = i32
        L.paged_multi_token_step.argtypes = [P, P, P, P, P, P, i32, i32, P, P, i32, i32, i32,
                                             ctypes.POINTER(CacheDesc), f32, P, P, P, sz, i32, P]
        L.pkv_copy_blocks.argtypes = [P, i32, ctypes.POINTER(CacheDesc), P, P, P]
        L.pkv_multi_token_kernel.restype = i32
        L.pkv_multi_token_kernel.argtypes = [i32, i32, i32, ctypes.POINTER(CacheDesc), i32]
        L.pkv_validate.restype = i32
        L.pkv_validate.argtypes = [P, P, i32, i32, P, i32, P, ctypes.POINTER(CacheDesc), P, P]
        L.pkv_probe_stream_read.restype = i32
        L.pkv_probe_stream_read.argtypes = [P, sz, P, i32, P]
        L.pkv_probe_gather_read.restype = i32
        L.pkv_probe_gather_read.argtypes = [P, sz, P, sz, P, i64, i32, P, i32, P]
        L.pkv_pool_create.restype = P
        L.pkv_pool_create.argtypes = [i32, i32]
        L.pkv_pool_create_with_free_list.restype = P
        L.pkv_pool_create_with_free_list.argtypes = [i32, i32, P, i32]
        L.pkv_pool_destroy.restype = None
        L.pkv_pool_destroy.argtypes = [P]
        L.pkv_pool_add_sequence.restype = i32
        L.pkv_pool_add_sequence.argtypes = [P, i64, i64]
        L.pkv_pool_append_slots.restype = i32
        L.pkv_pool_append_slots.argtypes = [P, P, i32, P, P, P]
        L.pkv_pool_fork.restype = i32
        L.pkv_pool_fork.argtypes = [P, i64, i64]
        L.pkv_pool_free.restype = i32
        L.pkv_pool_free.argtypes = [P, i64]
        L.pkv_pool_num_free.restype = i32
        L.pkv_pool_num_free.argtypes = [P]
        L.pkv_pool_ref_count.restype = i32
        L.pkv_pool_ref_count.argtypes = [P, i32]
        L.pkv_pool_seq_len.restype = i64
        L.pkv_pool_seq_len.argtypes = [P, i64]
        L.pkv_pool_block_table.restype = i32
        L.pkv_pool_block_table.argtypes = [P, i64, P, i32]
        L.pkv_pool_export.restype = i32
        L.pkv_pool_export.argtypes = [P, P, i32, i32, i32, P, P]
        _lib = L
    return _lib


def _check(func: str, status: int) -> None:
    if status != PKV_OK:
        raise PkvError(func, status, library())


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dev(t: torch.Tensor, name: str) -> int:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _sched(schedule: Optional[torch.Tensor]):
    if schedule is None:
        return None, 0
    return _dev(schedule, "schedule"), schedule.numel() * schedule.element_size()


def cache_desc(k_cache: torch.Tensor, v_cache: torch.Tensor, k_scale: float = 1.0,
               v_scale: float = 1.0) -> CacheDesc:
    """Descriptor of a key/value pool pair in the documented layouts (the
    scales matter only for FP8 pools: value = code * scale)."""
    if k_cache.dtype != v_cache.dtype or k_cache.dtype not in _DTYPES:
        raise ValueError("k_cache and v_cache must share dtype float32, bfloat16 or FP8 (uint8 codes)")
    if v_cache.dim() != 4 or k_cache.dim() != 5:
        raise ValueError("k_cache must be [nb, Hkv, hs/x, B, x] and v_cache [nb, Hkv, hs, B]")
    nb, hkv, hs, B = v_cache.shape
    x = 16 // k_cache.element_size()
    if tuple(k_cache.shape) != (nb, hkv, hs // x, B, x) or hs % x:
        raise ValueError(f"k_cache shape {tuple(k_cache.shape)} does not match v_cache {tuple(v_cache.shape)}")
    return CacheDesc(nb, hkv, B, hs, _DTYPES[k_cache.dtype], float(k_scale), float(v_scale), 0)


def io_dtype(k_cache: torch.Tensor) -> torch.dtype:
    """Element type of q, out and the appended k, v for these pools."""
    return torch.bfloat16 if _DTYPES.get(k_cache.dtype) == PKV_FP8_E4M3 else k_cache.dtype


def _out_tensor(q: torch.Tensor, out: Optional[torch.Tensor], out_dtype: Optional[torch.dtype],
                desc: CacheDesc) -> torch.Tensor:
    """The attention output: q's shape, and q's dtype or float32 (with bf16
    queries a float32 output receives the values before bf16 rounding; the
    descriptor's out_f32 is set for it)."""
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=q.device)
    if out.shape != q.shape or out.dtype not in (q.dtype, torch.float32):
        raise ValueError("out must have q's shape and q's dtype (or float32)")
    desc.out_f32 = 1 if out.dtype == torch.float32 else 0
    return out


def layout_version() -> int:
    return int(library().pkv_layout_version())


def decode_slot_mapping(block_tables: torch.Tensor, seq_lens: torch.Tensor, block_size: int,
                        out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """int64 [S]: slot of each sequence's newest token (position L-1); -1 when L <= 0."""
    if block_tables.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise ValueError("block_tables and seq_lens must be int32")
    S, M = block_tables.shape
    if out is None:
        out = torch.empty(S, dtype=torch.int64, device=block_tables.device)
    _check("pkv_decode_slot_mapping", library().pkv_decode_slot_mapping(
        _dev(block_tables, "block_tables"), _dev(seq_lens, "seq_lens"), S, M, block_size,
        _dev(out, "out"), _stream(stream)))
    return out


def kv_cache_append(k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor, k_cache: torch.Tensor,
                    v_cache: torch.Tensor, stream=None, k_scale: float = 1.0, v_scale: float = 1.0) -> None:
    """Write k[i], v[i] ([T, Hkv, hs]) into slot slot_mapping[i] of the pools (in place)."""
    desc = cache_desc(k_cache, v_cache, k_scale, v_scale)
    T = k.shape[0]
    if k.shape != v.shape or tuple(k.shape[1:]) != (desc.num_kv_heads, desc.head_size):
        raise ValueError("k and v must be [T, Hkv, head_size]")
    if k.dtype != io_dtype(k_cache) or v.dtype != io_dtype(k_cache):
        raise ValueError("k, v and the pools must share a dtype")
    if slot_mapping.dtype != torch.int64 or slot_mapping.shape != (T,):
        raise ValueError("slot_mapping must be int64 [T]")
    if T == 0:
        return
    _check("kv_cache_append", library().kv_cache_append(
        _dev(k, "k"), _dev(v, "v"), _dev(slot_mapping, "slot_mapping"), T, ctypes.byref(desc),
        _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _stream(stream)))


def decode_append(k: torch.Tensor, v: torch.Tensor, block_tables: torch.Tensor, seq_lens: torch.Tensor,
                  k_cache: torch.Tensor, v_cache: torch.Tensor, slot_mapping: Optional[torch.Tensor] = None,
                  schedule: Optional[torch.Tensor] = None, stream=None, k_scale: float = 1.0,
                  v_scale: float = 1.0) -> Optional[torch.Tensor]:
    """One launch: slot of each sequence's newest token from its table, then
    append k[s], v[s] there.  Writes the slots to slot_mapping if given, and
    the batch's longest-first schedule to `schedule` (from alloc_schedule) if
    given."""
    desc = cache_desc(k_cache, v_cache, k_scale, v_scale)
    S = k.shape[0]
    if k.shape != v.shape or tuple(k.shape[1:]) != (desc.num_kv_heads, desc.head_size):
        raise ValueError("k and v must be [S, Hkv, head_size]")
    if k.dtype != io_dtype(k_cache) or v.dtype != io_dtype(k_cache):
        raise ValueError("k, v and the pools must share a dtype")
    if block_tables.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise ValueError("block_tables and seq_lens must be int32")
    if block_tables.shape[0] != S or seq_lens.shape != (S,):
        raise ValueError("block_tables must be [S, M] and seq_lens [S]")
    if slot_mapping is not None and (slot_mapping.dtype != torch.int64 or slot_mapping.shape != (S,)):
        raise ValueError("slot_mapping must be int64 [S]")
    if S == 0:
        return slot_mapping
    _check("pkv_decode_append", library().pkv_decode_append(
        _dev(k, "k"), _dev(v, "v"), _dev(block_tables, "block_tables"), _dev(seq_lens, "seq_lens"), S,
        block_tables.shape[1], ctypes.byref(desc), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(slot_mapping, "slot_mapping") if slot_mapping is not None else None,
        *_sched(schedule), _stream(stream)))
    return slot_mapping


def decode_partition_tokens(num_seqs, num_q_heads, num_kv_heads, head_size, max_blocks_per_seq, block_size,
                            partition_tokens=0) -> int:
    return int(library().pkv_decode_partition_tokens(num_seqs, num_q_heads, num_kv_heads, head_size,
                                                     max_blocks_per_seq, block_size, partition_tokens))


def decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_size, max_blocks_per_seq, block_size,
                           partition_tokens=0) -> int:
    return int(library().pkv_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_size,
                                                    max_blocks_per_seq, block_size, partition_tokens))


def alloc_workspace(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, block_tables: torch.Tensor,
                    partition_tokens: int = 0) -> Optional[torch.Tensor]:
    desc = cache_desc(k_cache, v_cache)
    S, Hq, _ = q.shape
    n = decode_workspace_bytes(S, Hq, desc.num_kv_heads, desc.head_size, block_tables.shape[1], desc.block_size,
                               partition_tokens)
    if n == 0:
        return None
    return torch.empty(n, dtype=torch.uint8, device=q.device)


def schedule_bytes(num_seqs: int, max_blocks_per_seq: int) -> int:
    return int(library().pkv_decode_schedule_bytes(num_seqs, max_blocks_per_seq))


def alloc_schedule(block_tables: torch.Tensor) -> Optional[torch.Tensor]:
    """Device buffer for the longest-first schedule of a batch with these
    block tables (None when the batch takes none)."""
    n = schedule_bytes(block_tables.shape[0], block_tables.shape[1])
    if n == 0:
        return None
    return torch.empty(n, dtype=torch.uint8, device=block_tables.device)


def step_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_size, max_blocks_per_seq, block_size,
                         partition_tokens=0) -> int:
    return int(library().pkv_decode_step_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_size,
                                                         max_blocks_per_seq, block_size, partition_tokens))


def alloc_step_workspace(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                         block_tables: torch.Tensor, partition_tokens: int = 0) -> Optional[torch.Tensor]:
    desc = cache_desc(k_cache, v_cache)
    S, Hq, _ = q.shape
    n = step_workspace_bytes(S, Hq, desc.num_kv_heads, desc.head_size, block_tables.shape[1], desc.block_size,
                             partition_tokens)
    if n == 0:
        return None
    return torch.empty(n, dtype=torch.uint8, device=q.device)


def paged_decode_attention(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                           block_tables: torch.Tensor, seq_lens: torch.Tensor, scale: float,
                           out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                           partition_tokens: int = 0, schedule: Optional[torch.Tensor] = None,
                           stream=None, k_scale: float = 1.0, v_scale: float = 1.0,
                           out_dtype: Optional[torch.dtype] = None) -> torch.Tensor:
    """out[s, h] = softmax(scale * q[s, h] K^T) V over the L = seq_lens[s]
    tokens of sequence s, K/V found through block_tables.  `schedule`: the
    longest-first schedule decode_append wrote for these tables and lengths
    (optional; results are the same without it).  `out` (or out_dtype) may
    be float32 with bf16 queries: the values before bf16 rounding."""
    desc = cache_desc(k_cache, v_cache, k_scale, v_scale)
    if q.dtype != io_dtype(k_cache):
        raise ValueError("q must have the pools' dtype")
    S, Hq, hs = q.shape
    if hs != desc.head_size:
        raise ValueError("q head size does not match the pools")
    if block_tables.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise ValueError("block_tables and seq_lens must be int32")
    if block_tables.shape[0] != S or seq_lens.shape != (S,):
        raise ValueError("block_tables must be [S, M] and seq_lens [S]")
    M = block_tables.shape[1]
    out = _out_tensor(q, out, out_dtype, desc)
    if workspace is None:
        workspace = alloc_workspace(q, k_cache, v_cache, block_tables, partition_tokens)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("paged_decode_attention", library().paged_decode_attention(
        _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(block_tables, "block_tables"),
        _dev(seq_lens, "seq_lens"), S, Hq, M, ctypes.byref(desc), float(scale), _dev(out, "out"), ws_ptr, ws_bytes,
        int(partition_tokens), *_sched(schedule), _stream(stream)))
    return out


def paged_decode_step(q: torch.Tensor, new_k: torch.Tensor, new_v: torch.Tensor, k_cache: torch.Tensor,
                      v_cache: torch.Tensor, block_tables: torch.Tensor, seq_lens: torch.Tensor, scale: float,
                      out: Optional[torch.Tensor] = None, slot_mapping: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None, partition_tokens: int = 0,
                      stream=None, k_scale: float = 1.0, v_scale: float = 1.0,
                      out_dtype: Optional[torch.dtype] = None) -> torch.Tensor:
    """A whole decode step in one call: store new_k[s], new_v[s] at position
    seq_lens[s] - 1, then attend over all seq_lens[s] tokens.  The append
    launch also writes the batch's longest-first schedule into the workspace
    (see alloc_step_workspace) and the attention launch reads it.
    Bit-identical to decode_append followed by paged_decode_attention."""
    desc = cache_desc(k_cache, v_cache, k_scale, v_scale)
    if q.dtype != io_dtype(k_cache):
        raise ValueError("q must have the pools' dtype")
    S, Hq, hs = q.shape
    if hs != desc.head_size:
        raise ValueError("q head size does not match the pools")
    if new_k.shape != new_v.shape or tuple(new_k.shape) != (S, desc.num_kv_heads, desc.head_size):
        raise ValueError("new_k and new_v must be [S, Hkv, head_size]")
    if new_k.dtype != io_dtype(k_cache) or new_v.dtype != io_dtype(k_cache):
        raise ValueError("new_k, new_v and the pools must share a dtype")
    if block_tables.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise ValueError("block_tables and seq_lens must be int32")
    if block_tables.shape[0] != S or seq_lens.shape != (S,):
        raise ValueError("block_tables must be [S, M] and seq_lens [S]")
    if slot_mapping is not None and (slot_mapping.dtype != torch.int64 or slot_mapping.shape != (S,)):
        raise ValueError("slot_mapping must be int64 [S]")
    M = block_tables.shape[1]
    out = _out_tensor(q, out, out_dtype, desc)
    if workspace is None:
        workspace = alloc_step_workspace(q, k_cache, v_cache, block_tables, partition_tokens)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("paged_decode_step", library().paged_decode_step(
        _dev(q, "q"), _dev(new_k, "new_k"), _dev(new_v, "new_v"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(block_tables, "block_tables"), _dev(seq_lens, "seq_lens"), S, Hq, M, ctypes.byref(desc), float(scale),
        _dev(out, "out"), _dev(slot_mapping, "slot_mapping") if slot_mapping is not None else None, ws_ptr, ws_bytes,
        int(partition_tokens), _stream(stream)))
    return out


# Workspace size of the library's own device array (paged_decode_step_static).
STATIC_SCRATCH_BYTES = 32 << 20


def paged_decode_step_static(q: torch.Tensor, new_k: torch.Tensor, new_v: torch.Tensor, k_cache: torch.Tensor,
                             v_cache: torch.Tensor, block_tables: torch.Tensor, seq_lens: torch.Tensor, scale: float,
                             out: torch.Tensor, slot_mapping: Optional[torch.Tensor] = None,
                             partition_tokens: int = 0, stream=None, k_scale: float = 1.0,
                             v_scale: float = 1.0) -> torch.Tensor:
    """paged_decode_step without a workspace argument and without any
    allocation: the library takes the workspace from its own device array
    (STATIC_SCRATCH_BYTES per GPU).  `out` must be given (it may be float32
    with bf16 queries).  Calls that could overlap on one GPU must not be
    issued: they share the array."""
    desc = cache_desc(k_cache, v_cache, k_scale, v_scale)
    if q.dtype != io_dtype(k_cache):
        raise ValueError("q must have the pools' dtype")
    S, Hq, hs = q.shape
    if hs != desc.head_size:
        raise ValueError("q head size does not match the pools")
    if new_k.shape != new_v.shape or tuple(new_k.shape) != (S, desc.num_kv_heads, desc.head_size):
        raise ValueError("new_k and new_v must be [S, Hkv, head_size]")
    if new_k.dtype != io_dtype(k_cache) or new_v.dtype != io_dtype(k_cache):
        raise ValueError("new_k, new_v and the pools must share a dtype")
    if block_tables.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise ValueError("block_tables and seq_lens must be int32")
    if block_tables.shape[0] != S or seq_lens.shape != (S,):
        raise ValueError("block_tables must be [S, M] and seq_lens [S]")
    if slot_mapping is not None and (slot_mapping.dtype != torch.int64 or slot_mapping.shape != (S,)):
        raise ValueError("slot_mapping must be int64 [S]")
    if out is None:
        raise ValueError("out must be given (this call allocates nothing)")
    out = _out_tensor(q, out, None, desc)
    _check("paged_decode_step_static", library().paged_decode_step_static(
        _dev(q, "q"), _dev(new_k, "new_k"), _dev(new_v, "new_v"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(block_tables, "block_tables"), _dev(seq_lens, "seq_lens"), S, Hq, block_tables.shape[1],
        ctypes.byref(desc), float(scale), _dev(out, "out"),
        _dev(slot_mapping, "slot_mapping") if slot_mapping is not None else None, int(partition_tokens),
        _stream(stream)))
    return out


def decode_step(q, k_cache, v_cache, block_tables, seq_lens, new_k, new_v, scale, out=None, workspace=None,
                slot_mapping=None, partition_tokens=0, stream=None, k_scale=1.0, v_scale=1.0,
                out_dtype=None) -> torch.Tensor:
    """One decode step: append of the new tokens, then attention (two launches on one stream)."""
    return paged_decode_step(q, new_k, new_v, k_cache, v_cache, block_tables, seq_lens, scale, out=out,
                             slot_mapping=slot_mapping, workspace=workspace, partition_tokens=partition_tokens,
                             stream=stream, k_scale=k_scale, v_scale=v_scale, out_dtype=out_dtype)


# ---- several query tokens per sequence -------------------------------------
# partition_tokens: 0 = library's choice, > 0 = the partitioned kernel with
# that length, PARTITION_NONE = the unpartitioned (prefill) kernel.
PARTITION_NONE = -1

# Rows q_start[s] .. q_start[s+1]-1 of q / out / new k, v belong to sequence s
# and are its last n_s tokens; row i sits at position seq_lens[s] - n_s + i and
# attends causally.  max_q_len (>= every n_s) is a host int, so that no call
# waits for the device.

def multi_token_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_size, max_q_len, max_blocks_per_seq,
                                block_size, partition_tokens=0) -> int:
    return int(library().pkv_multi_token_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_size, max_q_len,
                                                         max_blocks_per_seq, block_size, partition_tokens))


def alloc_multi_token_workspace(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                                block_tables: torch.Tensor, max_q_len: int,
                                partition_tokens: int = 0) -> Optional[torch.Tensor]:
    desc = cache_desc(k_cache, v_cache)
    n = multi_token_workspace_bytes(block_tables.shape[0], q.shape[1], desc.num_kv_heads, desc.head_size, max_q_len,
                                    block_tables.shape[1], desc.block_size, partition_tokens)
    if n == 0:
        return None
    return torch.empty(n, dtype=torch.uint8, device=q.device)


def multi_token_kernel(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, block_tables: torch.Tensor,
                       max_q_len: int, partition_tokens: int = 0) -> str:
    """'unpartitioned' or 'partitioned': the kernel paged_multi_token_attention
    runs for these sizes."""
    desc = cache_desc(k_cache, v_cache)
    k = library().pkv_multi_token_kernel(block_tables.shape[0], q.shape[1], int(max_q_len), ctypes.byref(desc),
                                         int(partition_tokens))
    if k < 0:
        raise ValueError("these sizes are rejected by paged_multi_token_attention")
    return "unpartitioned" if k == 1 else "partitioned"


def multi_token_step_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_size, max_q_len, max_blocks_per_seq,
                                     block_size, partition_tokens=0) -> int:
    return int(library().pkv_multi_token_step_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_size,
                                                              max_q_len, max_blocks_per_seq, block_size,
                                                              partition_tokens))


def alloc_multi_token_step_workspace(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                                     block_tables: torch.Tensor, max_q_len: int,
                                     partition_tokens: int = 0) -> Optional[torch.Tensor]:
    """Workspace of paged_multi_token_step: the attention partials plus the
    batch's longest-first schedule."""
    desc = cache_desc(k_cache, v_cache)
    n = multi_token_step_workspace_bytes(block_tables.shape[0], q.shape[1], desc.num_kv_heads, desc.head_size,
                                         max_q_len, block_tables.shape[1], desc.block_size, partition_tokens)
    if n == 0:
        return None
    return torch.empty(n, dtype=torch.uint8, device=q.device)


def _check_rows(q, q_start, block_tables, seq_lens, desc, k_cache):
    if q.dtype != io_dtype(k_cache):
        raise ValueError("q must have the pools' dtype")
    if q.dim() != 3 or q.shape[2] != desc.head_size:
        raise ValueError("q must be [rows, Hq, head_size]")
    if block_tables.dtype != torch.int32 or seq_lens.dtype != torch.int32 or q_start.dtype != torch.int32:
        raise ValueError("block_tables, seq_lens and q_start must be int32")
    S = block_tables.shape[0]
    if seq_lens.shape != (S,) or q_start.shape != (S + 1,):
        raise ValueError("seq_lens must be [S] and q_start [S + 1]")
    return S


def multi_token_slot_mapping(block_tables: torch.Tensor, seq_lens: torch.Tensor, q_start: torch.Tensor,
                             num_q_rows: int, max_q_len: int, block_size: int, out: Optional[torch.Tensor] = None,
                             schedule: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """int64 [num_q_rows]: the slot of each query row's position.  Also
    writes the batch's longest-first schedule to `schedule` (from
    alloc_schedule) if given."""
    S = block_tables.shape[0]
    if out is None:
        out = torch.empty(num_q_rows, dtype=torch.int64, device=block_tables.device)
    if out.dtype != torch.int64 or out.shape != (num_q_rows,):
        raise ValueError("slot_mapping must be int64 [rows]")
    _check("pkv_multi_token_slot_mapping", library().pkv_multi_token_slot_mapping(
        _dev(block_tables, "block_tables"), _dev(seq_lens, "seq_lens"), _dev(q_start, "q_start"), S, num_q_rows,
        int(max_q_len), block_tables.shape[1], int(block_size), _dev(out, "slot_mapping"), *_sched(schedule),
        _stream(stream)))
    return out


def multi_token_append(k: torch.Tensor, v: torch.Tensor, q_start: torch.Tensor, max_q_len: int,
                       block_tables: torch.Tensor, seq_lens: torch.Tensor, k_cache: torch.Tensor,
                       v_cache: torch.Tensor, stream=None, k_scale: float = 1.0, v_scale: float = 1.0) -> None:
    """Stores k[r], v[r] ([rows, Hkv, hs]) of every query row in the slot of
    its position, block by block."""
    desc = cache_desc(k_cache, v_cache, k_scale, v_scale)
    if k.shape != v.shape or k.dim() != 3 or tuple(k.shape[1:]) != (desc.num_kv_heads, desc.head_size):
        raise ValueError("k and v must be [rows, Hkv, head_size]")
    if k.dtype != io_dtype(k_cache) or v.dtype != io_dtype(k_cache):
        raise ValueError("k, v and the pools must share a dtype")
    S = block_tables.shape[0]
    if q_start.dtype != torch.int32 or q_start.shape != (S + 1,):
        raise ValueError("q_start must be int32 [S + 1]")
    _check("pkv_multi_token_append", library().pkv_multi_token_append(
        _dev(k, "k"), _dev(v, "v"), _dev(q_start, "q_start"), k.shape[0], int(max_q_len),
        _dev(block_tables, "block_tables"), _dev(seq_lens, "seq_lens"), S, block_tables.shape[1],
        ctypes.byref(desc), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _stream(stream)))


def paged_multi_token_attention(q: torch.Tensor, q_start: torch.Tensor, max_q_len: int, k_cache: torch.Tensor,
                                v_cache: torch.Tensor, block_tables: torch.Tensor, seq_lens: torch.Tensor,
                                scale: float, out: Optional[torch.Tensor] = None,
                                workspace: Optional[torch.Tensor] = None, partition_tokens: int = 0,
                                schedule: Optional[torch.Tensor] = None, stream=None, k_scale: float = 1.0,
                                v_scale: float = 1.0, out_dtype: Optional[torch.dtype] = None) -> torch.Tensor:
    """Causal paged attention of every query row over its sequence's cached
    tokens (the rows' own tokens must already be in the cache).  `schedule`:
    the one multi_token_slot_mapping wrote for these tables and lengths, or
    None."""
    desc = cache_desc(k_cache, v_cache, k_scale, v_scale)
    S = _check_rows(q, q_start, block_tables, seq_lens, desc, k_cache)
    rows, Hq, _ = q.shape
    out = _out_tensor(q, out, out_dtype, desc)
    if workspace is None:
        workspace = alloc_multi_token_workspace(q, k_cache, v_cache, block_tables, max_q_len, partition_tokens)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("paged_multi_token_attention", library().paged_multi_token_attention(
        _dev(q, "q"), _dev(q_start, "q_start"), rows, int(max_q_len), _dev(k_cache, "k_cache"),
        _dev(v_cache, "v_cache"), _dev(block_tables, "block_tables"), _dev(seq_lens, "seq_lens"), S, Hq,
        block_tables.shape[1], ctypes.byref(desc), float(scale), _dev(out, "out"), ws_ptr, ws_bytes,
        int(partition_tokens), *_sched(schedule), _stream(stream)))
    return out


def paged_multi_token_step(q: torch.Tensor, new_k: torch.Tensor, new_v: torch.Tensor, k_cache: torch.Tensor,
                           v_cache: torch.Tensor, q_start: torch.Tensor, max_q_len: int, block_tables: torch.Tensor,
                           seq_lens: torch.Tensor, scale: float, out: Optional[torch.Tensor] = None,
                           slot_mapping: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                           partition_tokens: int = 0, stream=None, k_scale: float = 1.0,
                           v_scale: float = 1.0, out_dtype: Optional[torch.dtype] = None) -> torch.Tensor:
    """Slot mapping of the rows, append of every row's new_k / new_v, then
    paged_multi_token_attention (three launches on one stream)."""
    desc = cache_desc(k_cache, v_cache, k_scale, v_scale)
    S = _check_rows(q, q_start, block_tables, seq_lens, desc, k_cache)
    rows, Hq, _ = q.shape
    if new_k.shape != new_v.shape or tuple(new_k.shape) != (rows, desc.num_kv_heads, desc.head_size):
        raise ValueError("new_k and new_v must be [rows, Hkv, head_size]")
    if new_k.dtype != io_dtype(k_cache) or new_v.dtype != io_dtype(k_cache):
        raise ValueError("new_k, new_v and the pools must share a dtype")
    if slot_mapping is None:
        slot_mapping = torch.empty(rows, dtype=torch.int64, device=q.device)
    if slot_mapping.dtype != torch.int64 or slot_mapping.shape != (rows,):
        raise ValueError("slot_mapping must be int64 [rows]")
    out = _out_tensor(q, out, out_dtype, desc)
    if workspace is None:
        workspace = alloc_multi_token_step_workspace(q, k_cache, v_cache, block_tables, max_q_len,
                                                     partition_tokens)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("paged_multi_token_step", library().paged_multi_token_step(
        _dev(q, "q"), _dev(new_k, "new_k"), _dev(new_v, "new_v"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(q_start, "q_start"), rows, int(max_q_len), _dev(block_tables, "block_tables"), _dev(seq_lens, "seq_lens"),
        S, Hq, block_tables.shape[1], ctypes.byref(desc), float(scale), _dev(out, "out"),
        _dev(slot_mapping, "slot_mapping"), ws_ptr, ws_bytes, int(partition_tokens), _stream(stream)))
    return out


# Fields of pkv_validate_report, in order (int64 each).
VALIDATE_FIELDS = ("bad_seq_lens", "bad_block_ids", "bad_slots", "duplicate_slots", "shared_block_writes",
                   "first_bad_seq_len", "first_bad_block_id", "first_bad_slot", "first_duplicate_slot",
                   "first_shared_block_write")


def validate(block_tables: torch.Tensor, seq_lens: torch.Tensor, num_blocks: int, block_size: int,
             slot_mapping: Optional[torch.Tensor] = None, ref_counts: Optional[torch.Tensor] = None,
             stream=None) -> dict:
    """Checks tables, lengths and slots against the kernels' device-side
    contract for a pool of num_blocks blocks of block_size tokens (block IDs
    in the pool, lengths within the table, distinct slots inside the pool, no
    slot in a block with ref_counts > 1) and returns the report as a dict of
    VALIDATE_FIELDS (first_* = -1 when none).  Without slot_mapping the
    decode step's slots are checked.  Reads no pool data; waits for the GPU
    to return the report."""
    # only the pool's block count and block size matter to the check
    desc = CacheDesc(int(num_blocks), 1, int(block_size), 128, PKV_BF16, 1.0, 1.0, 0)
    if block_tables.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise ValueError("block_tables and seq_lens must be int32")
    S, M = block_tables.shape
    if seq_lens.shape != (S,):
        raise ValueError("seq_lens must be [S]")
    if slot_mapping is not None and (slot_mapping.dtype != torch.int64 or slot_mapping.dim() != 1):
        raise ValueError("slot_mapping must be int64 [T]")
    if ref_counts is not None and (ref_counts.dtype != torch.int32 or ref_counts.shape != (desc.num_blocks,)):
        raise ValueError("ref_counts must be int32 [num_blocks]")
    report = torch.empty(len(VALIDATE_FIELDS), dtype=torch.int64, device=block_tables.device)
    _check("pkv_validate", library().pkv_validate(
        _dev(block_tables, "block_tables"), _dev(seq_lens, "seq_lens"), S, M,
        _dev(slot_mapping, "slot_mapping") if slot_mapping is not None else None,
        slot_mapping.shape[0] if slot_mapping is not None else 0,
        _dev(ref_counts, "ref_counts") if ref_counts is not None else None, ctypes.byref(desc),
        _dev(report, "report"), _stream(stream)))
    torch.cuda.synchronize(report.device)
    return dict(zip(VALIDATE_FIELDS, report.cpu().tolist()))


def probe_stream_read(buf: torch.Tensor, out: torch.Tensor, work_groups: int, stream=None) -> None:
    """One streaming read of the whole of `buf` (a measurement aid: time it to
    get the GPU's practical read bandwidth); `out` is a 4-byte device buffer."""
    if not buf.is_contiguous() or (buf.numel() * buf.element_size()) % 16 != 0:
        raise ValueError("buf must be contiguous and a multiple of 16 bytes")
    if out.numel() * out.element_size() < 4:
        raise ValueError("out must hold 4 bytes")
    _check("pkv_probe_stream_read", library().pkv_probe_stream_read(
        _dev(buf, "buf"), buf.numel() * buf.element_size(), _dev(out, "out"), int(work_groups), _stream(stream)))


def probe_gather_read(buf0: torch.Tensor, buf1: torch.Tensor, tile_offsets: torch.Tensor, tile_bytes: int,
                      out: torch.Tensor, work_groups: int, stream=None) -> None:
    """One read of the tiles listed in tile_offsets (int64 byte offsets; even
    entries in buf0, odd ones in buf1), a measurement aid: time it to get
    the rate of a paged access pattern; `out` is a 4-byte device buffer."""
    for name, b in (("buf0", buf0), ("buf1", buf1)):
        if not b.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if tile_offsets.dtype != torch.int64 or not tile_offsets.is_contiguous():
        raise ValueError("tile_offsets must be a contiguous int64 tensor")
    if out.numel() * out.element_size() < 4:
        raise ValueError("out must hold 4 bytes")
    n = tile_offsets.numel()
    _check("pkv_probe_gather_read", library().pkv_probe_gather_read(
        _dev(buf0, "buf0"), buf0.numel() * buf0.element_size(), _dev(buf1, "buf1"),
        buf1.numel() * buf1.element_size(), _dev(tile_offsets, "tile_offsets") if n else None, n, int(tile_bytes),
        _dev(out, "out"), int(work_groups), _stream(stream)))


def copy_blocks(pairs: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, stream=None) -> None:
    """Copy whole blocks (every KV head, both pools): pairs is a device int32
    [n, 2] tensor of (src, dst) block ids; the dst blocks must be distinct
    and must not be sources of the same call."""
    desc = cache_desc(k_cache, v_cache)
    if pairs.dtype != torch.int32 or pairs.dim() != 2 or pairs.shape[1] != 2:
        raise ValueError("pairs must be int32 [n, 2]")
    n = pairs.shape[0]
    if n == 0:
        return
    _check("pkv_copy_blocks", library().pkv_copy_blocks(_dev(pairs.contiguous(), "pairs"), n, ctypes.byref(desc),
                                                        _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                                                        _stream(stream)))


class OutOfBlocks(RuntimeError):
    """The block pool has no free block left (nothing was changed)."""


class BlockPool:
    """Host block pool of the library (native code): free list, reference
    counts, block tables, fork and copy-on-write.  Sequence ids are ints."""

    def __init__(self, num_blocks: int, block_size: int, free_list=None):
        L = library()
        if free_list is None:
            h = L.pkv_pool_create(num_blocks, block_size)
        else:
            arr = (ctypes.c_int32 * len(free_list))(*free_list)
            h = L.pkv_pool_create_with_free_list(num_blocks, block_size, ctypes.cast(arr, ctypes.c_void_p),
                                                 len(free_list))
        if not h:
            raise ValueError("invalid pool arguments")
        self._h = ctypes.c_void_p(h)
        self._lib = L
        self.num_blocks = num_blocks
        self.block_size = block_size

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            self._lib.pkv_pool_destroy(h)
            self._h = None

    def _st(self, func: str, status: int) -> None:
        if status == PKV_ERR_OUT_OF_BLOCKS:
            raise OutOfBlocks(func)
        _check(func, status)

    def add_sequence(self, seq: int, num_tokens: int) -> None:
        self._st("pkv_pool_add_sequence", self._lib.pkv_pool_add_sequence(self._h, seq, num_tokens))

    def append_slots(self, seqs):
        """Reserve the next slot of each sequence.  Returns (slots, copies):
        a list of slots and a list of (src, dst) block copies to do first."""
        n = len(seqs)
        ids = (ctypes.c_int64 * max(n, 1))(*seqs)
        slots = (ctypes.c_int64 * max(n, 1))()
        copies = (ctypes.c_int32 * max(2 * n, 1))()
        nc = ctypes.c_int32(0)
        self._st("pkv_pool_append_slots", self._lib.pkv_pool_append_slots(
            self._h, ctypes.cast(ids, ctypes.c_void_p), n, ctypes.cast(slots, ctypes.c_void_p),
            ctypes.cast(copies, ctypes.c_void_p), ctypes.byref(nc)))
        return list(slots[:n]), [(copies[2 * i], copies[2 * i + 1]) for i in range(nc.value)]

    def append_slot(self, seq: int):
        slots, copies = self.append_slots([seq])
        return slots[0], (copies[0] if copies else None)

    def fork(self, parent: int, child: int) -> None:
        self._st("pkv_pool_fork", self._lib.pkv_pool_fork(self._h, parent, child))

    def free(self, seq: int) -> None:
        self._st("pkv_pool_free", self._lib.pkv_pool_free(self._h, seq))

    def num_free(self) -> int:
        return self._lib.pkv_pool_num_free(self._h)

    def ref_count(self, block: int) -> int:
        return self._lib.pkv_pool_ref_count(self._h, block)

    def seq_len(self, seq: int) -> int:
        return self._lib.pkv_pool_seq_len(self._h, seq)

    def table(self, seq: int):
        n = self._lib.pkv_pool_block_table(self._h, seq, None, 0)
        if n < 0:
            raise KeyError(seq)
        buf = (ctypes.c_int32 * max(n, 1))()
        self._lib.pkv_pool_block_table(self._h, seq, ctypes.cast(buf, ctypes.c_void_p), n)
        return list(buf[:n])

    def export(self, seqs, max_blocks_per_seq: int, pad_block: int = 0):
        """(block_tables int32 [S, M], seq_lens int32 [S]) as host tensors."""
        n = len(seqs)
        ids = (ctypes.c_int64 * max(n, 1))(*seqs)
        bt = torch.empty((n, max_blocks_per_seq), dtype=torch.int32)
        sl = torch.empty((n,), dtype=torch.int32)
        _check("pkv_pool_export", self._lib.pkv_pool_export(
            self._h, ctypes.cast(ids, ctypes.c_void_p), n, max_blocks_per_seq, pad_block, bt.data_ptr(),
            sl.data_ptr()))
        return bt, sl
