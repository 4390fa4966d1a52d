"""The C ABI without a GPU: the library loads, exports every function the
header declares, and rejects bad arguments on the host before any launch."""
import ctypes
import os
import re

import pytest

import paged_kv_cache_35_amd as pkv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pkv.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, -1, -2, -3


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"PKV_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pkv.LIB_PATH):
        pytest.fail("libpkv.so is not built (run __graft_entry__.build())")
    return pkv.library()


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("paged_decode_attention", "kv_cache_append", "pkv_decode_slot_mapping",
              "pkv_decode_workspace_bytes", "pkv_decode_partition_tokens", "pkv_status_string",
              "pkv_layout_version", "pkv_last_hip_error", "paged_decode_step", "pkv_decode_append",
              "pkv_decode_schedule_bytes", "pkv_decode_step_workspace_bytes", "paged_multi_token_attention",
              "pkv_multi_token_step_workspace_bytes", "pkv_multi_token_slot_mapping"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(pkv.LIB_PATH)
    for name in declared_functions():
        assert hasattr(raw, name), f"{name} declared in pkv.h but not exported"


def test_status_strings_and_layout(lib):
    assert lib.pkv_status_string(OK) == b"PKV_OK"
    assert lib.pkv_status_string(WORKSPACE) == b"PKV_ERR_WORKSPACE"
    assert lib.pkv_layout_version() == 2
    assert lib.pkv_status_string(-5) == b"PKV_ERR_OUT_OF_BLOCKS"


def desc(nb=32, hkv=8, B=16, hs=64, dtype=0, k_scale=1.0, v_scale=1.0):
    return pkv.CacheDesc(nb, hkv, B, hs, dtype, k_scale, v_scale)


FAKE = ctypes.c_void_p(0x10000)  # aligned, never dereferenced: validation fails first


def attn(lib, *, q=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, sl=FAKE, S=4, Hq=8, M=4, d=None, out=FAKE, ws=None,
         ws_bytes=0, P=0, sched=None, sched_bytes=0, scale=0.125):
    d = d or desc()
    return lib.paged_decode_attention(q, kc, vc, bt, sl, S, Hq, M, ctypes.byref(d), scale, out, ws, ws_bytes, P,
                                      sched, sched_bytes, None)


def test_attention_rejects_bad_arguments(lib):
    assert attn(lib, q=None) == INVALID
    assert attn(lib, out=None) == INVALID
    assert attn(lib, Hq=12) == INVALID                      # Hq % Hkv != 0
    assert attn(lib, Hq=8 * 32, d=desc(hkv=8)) == UNSUPPORTED  # group of 32 query heads
    assert attn(lib, d=desc(hs=96)) == UNSUPPORTED
    assert attn(lib, d=desc(B=4)) == UNSUPPORTED
    assert attn(lib, d=desc(B=128)) == UNSUPPORTED
    assert attn(lib, d=desc(B=8, dtype=2)) == UNSUPPORTED  # FP8 pools need B >= 16
    assert attn(lib, d=desc(dtype=7)) == UNSUPPORTED
    # FP8 pools need positive finite scales
    assert attn(lib, d=desc(dtype=2, k_scale=0.0)) == INVALID
    assert attn(lib, d=desc(dtype=2, v_scale=float("inf"))) == INVALID
    assert attn(lib, d=desc(dtype=2), S=0) == OK
    # the softmax scale must be positive and finite
    for bad in (0.0, -0.125, float("inf"), float("nan")):
        assert attn(lib, scale=bad) == INVALID
        assert attn(lib, scale=bad, S=0) == INVALID
    assert attn(lib, d=desc(nb=0)) == INVALID
    assert attn(lib, M=0) == INVALID
    assert attn(lib, S=-1) == INVALID
    assert attn(lib, q=ctypes.c_void_p(0x10008)) == INVALID   # misaligned
    assert attn(lib, P=24) == INVALID                        # not a multiple of B
    assert attn(lib, P=16 * 65) == INVALID                   # more than 64 blocks per partition
    assert attn(lib, M=0x7FFFFFFF) == INVALID                # M * B overflows
    # a long table needs a workspace
    assert attn(lib, M=4096) == WORKSPACE
    need = lib.pkv_decode_workspace_bytes(4, 8, 8, 64, 4096, 16, 0)
    assert attn(lib, M=4096, ws=FAKE, ws_bytes=need - 1) == WORKSPACE
    # a schedule buffer that is too small or misaligned
    need = lib.pkv_decode_schedule_bytes(4, 4)
    assert attn(lib, sched=FAKE, sched_bytes=need - 1) == WORKSPACE
    assert attn(lib, sched=ctypes.c_void_p(0x10004), sched_bytes=need) == WORKSPACE
    # nothing to do: valid no-op without touching the GPU
    assert attn(lib, S=0) == OK


def test_workspace_and_partition_sizes(lib):
    # one partition covers a short table: no workspace
    assert lib.pkv_decode_partition_tokens(4, 8, 8, 64, 4, 16, 0) == 64
    assert lib.pkv_decode_workspace_bytes(4, 8, 8, 64, 4, 16, 0) == 0
    # 512-token partitions by default, merged in chunks of 4 per work-group:
    # 128 blocks of 16 -> 4 partitions -> one chunk, no workspace
    assert lib.pkv_decode_partition_tokens(64, 32, 32, 128, 128, 16, 0) == 512
    assert lib.pkv_decode_workspace_bytes(64, 32, 32, 128, 128, 16, 0) == 0
    assert lib.pkv_decode_workspace_bytes(64, 32, 32, 128, 1024, 16, 0) == 64 * 32 * 8 * 130 * 4
    # explicit partition length: 4096 blocks of 32 in 512-token partitions -> 256 partitions, 64 chunks
    assert lib.pkv_decode_partition_tokens(8, 64, 8, 128, 4096, 32, 512) == 512
    assert lib.pkv_decode_workspace_bytes(8, 64, 8, 128, 4096, 32, 512) == 8 * 64 * 64 * 130 * 4
    assert lib.pkv_decode_partition_tokens(8, 64, 8, 128, 4096, 32, 48) == 0


def test_schedule_and_step_workspace_sizes(lib):
    # order[S], lens[S] and tables[S][M], each rounded up to 16 bytes, then
    # a 16-byte count and the chunk list [S][ceil(M / 4)] of uint32 pairs
    def sched(S, M):
        return 2 * (-(-S * 4 // 16) * 16) + (-(-S * M * 4 // 16) * 16) + 16 + S * (-(-M // 4)) * 8
    assert lib.pkv_decode_schedule_bytes(64, 128) == 2 * 256 + 64 * 128 * 4 + 16 + 64 * 32 * 8
    assert lib.pkv_decode_schedule_bytes(5, 3) == 2 * 32 + 64 + 16 + 5 * 1 * 8
    assert lib.pkv_decode_schedule_bytes(4096, 8) == sched(4096, 8)
    # no schedule for a single sequence or above 4096 sequences
    assert lib.pkv_decode_schedule_bytes(1, 128) == 0
    assert lib.pkv_decode_schedule_bytes(4097, 8) == 0
    # step = attention partials rounded up to 256 bytes + schedule
    assert lib.pkv_decode_step_workspace_bytes(64, 32, 32, 128, 128, 16, 0) == sched(64, 128)
    attn = 64 * 32 * 8 * 130 * 4
    assert lib.pkv_decode_step_workspace_bytes(64, 32, 32, 128, 1024, 16, 0) == attn + sched(64, 1024)
    assert lib.pkv_decode_step_workspace_bytes(1, 8, 8, 64, 4, 16, 0) == 0


def test_append_rejects_bad_arguments(lib):
    d = desc()
    f = lib.kv_cache_append
    assert f(FAKE, FAKE, FAKE, 4, None, FAKE, FAKE, None) == INVALID
    assert f(None, FAKE, FAKE, 4, ctypes.byref(d), FAKE, FAKE, None) == INVALID
    assert f(FAKE, FAKE, None, 4, ctypes.byref(d), FAKE, FAKE, None) == INVALID
    assert f(FAKE, FAKE, FAKE, -1, ctypes.byref(d), FAKE, FAKE, None) == INVALID
    assert f(FAKE, FAKE, FAKE, 4, ctypes.byref(d), None, FAKE, None) == INVALID
    assert f(FAKE, FAKE, FAKE, 4, ctypes.byref(desc(hs=80)), FAKE, FAKE, None) == UNSUPPORTED
    assert f(ctypes.c_void_p(0x10004), FAKE, FAKE, 4, ctypes.byref(d), FAKE, FAKE, None) == INVALID
    assert f(None, None, None, 0, ctypes.byref(d), FAKE, FAKE, None) == OK


def test_slot_mapping_rejects_bad_arguments(lib):
    f = lib.pkv_decode_slot_mapping
    assert f(None, FAKE, 4, 4, 16, FAKE, None) == INVALID
    assert f(FAKE, FAKE, 4, 0, 16, FAKE, None) == INVALID
    assert f(FAKE, FAKE, 4, 4, 0, FAKE, None) == INVALID
    assert f(None, None, 0, 4, 16, None, None) == OK


def test_binding_refuses_host_tensors():
    import torch

    q = torch.zeros(2, 4, 64)
    kc = torch.zeros(8, 4, 16, 16, 4)
    vc = torch.zeros(8, 4, 64, 16)
    bt = torch.zeros(2, 2, dtype=torch.int32)
    sl = torch.ones(2, dtype=torch.int32)
    with pytest.raises(ValueError):
        pkv.paged_decode_attention(q, kc, vc, bt, sl, 0.125, out=torch.zeros_like(q), workspace=None)
    with pytest.raises(ValueError):
        pkv.cache_desc(kc, vc[:, :, :32])


def test_step_requires_the_new_token(lib):
    d = desc()
    f = lib.paged_decode_step
    assert f(FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, 4, ctypes.byref(d), 0.125, FAKE, None, None, 0, 0,
             None) == INVALID
    assert f(FAKE, FAKE, ctypes.c_void_p(0x10002), FAKE, FAKE, FAKE, FAKE, 4, 8, 4, ctypes.byref(d), 0.125, FAKE,
             None, None, 0, 0, None) == INVALID
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, 4096, ctypes.byref(d), 0.125, FAKE, None, None, 0, 0,
             None) == WORKSPACE
    # a batch of 4 takes a schedule, so the step needs a workspace
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, 4, ctypes.byref(d), 0.125, FAKE, None, None, 0, 0,
             None) == WORKSPACE
    assert f(None, None, None, FAKE, FAKE, None, None, 0, 8, 4, ctypes.byref(d), 0.125, None, None, None, 0, 0,
             None) == OK


def test_decode_append_rejects_a_small_schedule(lib):
    d = desc()
    f = lib.pkv_decode_append
    need = lib.pkv_decode_schedule_bytes(4, 4)
    assert f(FAKE, FAKE, FAKE, FAKE, 4, 4, ctypes.byref(d), FAKE, FAKE, None, FAKE, need - 1, None) == WORKSPACE
    assert f(FAKE, FAKE, FAKE, FAKE, 0, 4, ctypes.byref(d), FAKE, FAKE, None, FAKE, 0, None) == OK


def test_multi_token_attention_rejects_a_small_schedule(lib):
    need = lib.pkv_decode_schedule_bytes(4, 4)
    f = lib.paged_multi_token_attention
    assert f(FAKE, FAKE, 8, 2, FAKE, FAKE, FAKE, FAKE, 4, 8, 4, ctypes.byref(desc()), 0.125, FAKE, None, 0, 0, FAKE,
             need - 1, None) == WORKSPACE


def test_multi_token_step_workspace_sizes(lib):
    f = lib.pkv_multi_token_step_workspace_bytes
    attn = lib.pkv_multi_token_workspace_bytes
    sched = lib.pkv_decode_schedule_bytes
    # partials rounded up to 256, then the schedule
    a = attn(256, 32, 8, 128, 4, 1024, 16, 0)
    assert a > 0 and f(256, 32, 8, 128, 4, 1024, 16, 0) == (a + 255) // 256 * 256 + sched(256, 1024)
    # no partials (one chunk covers the table): the schedule alone
    assert attn(64, 32, 32, 128, 8, 128, 16, 0) == 0
    assert f(64, 32, 32, 128, 8, 128, 16, 0) == sched(64, 128)
    # no schedule: one sequence or more than 4096
    assert f(1, 32, 8, 128, 4, 1024, 16, 0) == attn(1, 32, 8, 128, 4, 1024, 16, 0)
    assert f(4097, 32, 8, 128, 4, 8, 16, 0) == attn(4097, 32, 8, 128, 4, 8, 16, 0)
    # the unpartitioned kernel: no partials, the schedule alone
    assert f(16, 32, 8, 128, 512, 1024, 16, -1) == sched(16, 1024)
    # invalid shapes: 0
    assert f(16, 30, 8, 128, 4, 1024, 16, 0) == 0
    assert f(16, 32, 8, 128, 0, 1024, 16, 0) == 0


def test_multi_token_kernel_choice(lib):
    f = lib.pkv_multi_token_kernel
    bf16 = desc(hkv=8, hs=128, dtype=1)
    # 512 query tokens x G = 4 on 256 sequences: the unpartitioned kernel
    assert f(256, 32, 512, ctypes.byref(bf16), 0) == 1
    # 4 draft tokens (16 rows per KV head): the partitioned kernel
    assert f(256, 32, 4, ctypes.byref(bf16), 0) == 0
    # too few work-groups (2 sequences x 8 KV heads x 16 row blocks)
    assert f(2, 32, 512, ctypes.byref(bf16), 0) == 0
    # a requested partition length always selects the partitioned kernel
    assert f(256, 32, 512, ctypes.byref(bf16), 512) == 0
    # PKV_PARTITION_NONE: the unpartitioned kernel where it is supported
    assert f(4, 32, 4, ctypes.byref(bf16), -1) == 1
    assert f(4, 32, 4, ctypes.byref(desc(hkv=8, hs=128, dtype=0)), -1) == -1   # fp32 pools
    assert f(4, 32, 4, ctypes.byref(desc(hkv=8, hs=128, B=8, dtype=1)), -1) == -1
    assert f(256, 32, 512, ctypes.byref(desc(hkv=8, hs=128, dtype=0)), 0) == 0  # fp32: partitioned
    # rejected sizes
    assert f(4, 30, 4, ctypes.byref(bf16), 0) == -1
    assert f(4, 32, 4, None, 0) == -1
    assert f(4, 32, 4, ctypes.byref(bf16), -2) == -1


def test_stream_probe_rejects_bad_arguments(lib):
    f = lib.pkv_probe_stream_read
    assert f(None, 1024, FAKE, 64, None) == INVALID
    assert f(FAKE, 1024, None, 64, None) == INVALID
    assert f(ctypes.c_void_p(0x10008), 1024, FAKE, 64, None) == INVALID
    assert f(FAKE, 1000, FAKE, 64, None) == INVALID
    assert f(FAKE, 1024, FAKE, 0, None) == INVALID
    assert f(FAKE, 1024, FAKE, (1 << 20) + 1, None) == INVALID
    assert f(FAKE, 0, FAKE, 64, None) == OK  # nothing to read


def test_gather_probe_rejects_bad_arguments(lib):
    f = lib.pkv_probe_gather_read
    assert f(None, 4096, FAKE, 4096, FAKE, 4, 1024, FAKE, 8, None) == INVALID
    assert f(FAKE, 4096, None, 4096, FAKE, 4, 1024, FAKE, 8, None) == INVALID
    assert f(FAKE, 4096, FAKE, 4096, FAKE, 4, 1024, None, 8, None) == INVALID
    assert f(ctypes.c_void_p(0x10008), 4096, FAKE, 4096, FAKE, 4, 1024, FAKE, 8, None) == INVALID
    assert f(FAKE, 4096, FAKE, 4096, None, 4, 1024, FAKE, 8, None) == INVALID   # tiles without a list
    assert f(FAKE, 4096, FAKE, 4096, FAKE, -1, 1024, FAKE, 8, None) == INVALID
    for tb in (0, 512, 1536, (1 << 20) + 1024):
        assert f(FAKE, 4096, FAKE, 4096, FAKE, 4, tb, FAKE, 8, None) == INVALID
    assert f(FAKE, 4096, FAKE, 4096, FAKE, 4, 1024, FAKE, 0, None) == INVALID
    assert f(FAKE, 4096, FAKE, 4096, FAKE, 4, 1024, FAKE, (1 << 20) + 1, None) == INVALID
    assert f(FAKE, 4096, FAKE, 4096, None, 0, 1024, FAKE, 8, None) == OK  # nothing to read


def test_multi_token_workspace_sizes(lib):
    f = lib.pkv_multi_token_workspace_bytes
    # one chunk covers the table: none
    assert f(4, 8, 8, 64, 16, 4, 16, 0) == 0
    # 1024 blocks of 16 in 512-token partitions: 32 partitions, 8 chunks;
    # 4 query tokens x G = 4 -> one 16-row tile per (sequence, KV head)
    assert f(256, 32, 8, 128, 4, 1024, 16, 0) == 256 * 8 * 1 * 8 * 16 * 130 * 4
    # 512 tokens x G = 4 -> 128 tiles
    assert f(16, 32, 8, 128, 512, 1024, 16, 0) == 16 * 8 * 128 * 8 * 16 * 130 * 4
    assert f(16, 32, 8, 128, 0, 1024, 16, 0) == 0
    assert f(16, 30, 8, 128, 4, 1024, 16, 0) == 0


def mq(lib, *, q=FAKE, qs=FAKE, rows=8, mql=2, S=4, Hq=8, M=4, d=None, out=FAKE, ws=None, ws_bytes=0, P=0,
       scale=0.125):
    d = d or desc()
    return lib.paged_multi_token_attention(q, qs, rows, mql, FAKE, FAKE, FAKE, FAKE, S, Hq, M, ctypes.byref(d),
                                           scale, out, ws, ws_bytes, P, None, 0, None)


def test_multi_token_attention_rejects_bad_arguments(lib):
    assert mq(lib, qs=None) == INVALID
    assert mq(lib, rows=-1) == INVALID
    assert mq(lib, mql=-1) == INVALID
    assert mq(lib, mql=65536) == UNSUPPORTED
    assert mq(lib, q=ctypes.c_void_p(0x10008)) == INVALID
    assert mq(lib, Hq=12) == INVALID
    for bad in (0.0, -1.0, float("nan")):
        assert mq(lib, scale=bad) == INVALID
        assert mq(lib, scale=bad, P=-1) == INVALID
    need = lib.pkv_multi_token_workspace_bytes(4, 8, 8, 64, 2, 4096, 16, 0)
    assert need > 0
    assert mq(lib, M=4096, ws=FAKE, ws_bytes=need - 1) == WORKSPACE
    # the decode workspace of the same shape is smaller: still refused
    dec = lib.pkv_decode_workspace_bytes(4, 8, 8, 64, 4096, 16, 0)
    assert 0 < dec < need
    assert mq(lib, M=4096, ws=FAKE, ws_bytes=dec) == WORKSPACE
    # nothing to do
    assert lib.paged_multi_token_attention(None, None, 0, 0, None, None, None, None, 0, 8, 4, ctypes.byref(desc()),
                                           0.125, None, None, 0, 0, None, 0, None) == OK


def test_multi_token_calls_without_rows_do_nothing(lib):
    # sequences that all sit this step out: no rows, so q, out and the new
    # rows are empty (null); the shapes are still checked
    for rows, mql in ((0, 0), (0, 4), (8, 0)):
        assert mq(lib, q=None, out=None, rows=rows, mql=mql) == OK
        assert mq(lib, q=None, out=None, rows=rows, mql=mql, Hq=12) == INVALID
        assert lib.paged_multi_token_step(None, None, None, FAKE, FAKE, FAKE, rows, mql, FAKE, FAKE, 4, 8, 4,
                                          ctypes.byref(desc()), 0.125, None, None, None, 0, 0, None) == OK
        assert lib.paged_multi_token_step(None, None, None, FAKE, FAKE, FAKE, rows, mql, FAKE, FAKE, 4, 8, 4,
                                          ctypes.byref(desc(hs=96)), 0.125, None, None, None, 0, 0, None) != OK


def test_multi_token_step_and_slot_mapping_reject_bad_arguments(lib):
    d = desc()
    f = lib.paged_multi_token_step
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8, 2, FAKE, FAKE, 4, 8, 4, ctypes.byref(d), 0.125, FAKE, FAKE, None, 0,
            0, None]
    for i, bad in ((1, None), (2, ctypes.c_void_p(0x10002)), (16, None)):
        a = list(args)
        a[i] = bad
        assert f(*a) == INVALID
    g = lib.pkv_multi_token_slot_mapping
    assert g(FAKE, FAKE, None, 4, 8, 2, 4, 16, FAKE, None, 0, None) == INVALID
    assert g(FAKE, FAKE, FAKE, 4, 8, 2, 0, 16, FAKE, None, 0, None) == INVALID
    assert g(FAKE, FAKE, FAKE, 70000, 8, 2, 4, 16, FAKE, None, 0, None) == UNSUPPORTED
    assert g(None, None, None, 0, 0, 0, 4, 16, None, None, 0, None) == OK
    # a schedule buffer that is too small or misaligned
    need = lib.pkv_decode_schedule_bytes(4, 4)
    assert g(FAKE, FAKE, FAKE, 4, 8, 2, 4, 16, FAKE, FAKE, need - 1, None) == WORKSPACE
    assert g(FAKE, FAKE, FAKE, 4, 8, 2, 4, 16, FAKE, ctypes.c_void_p(0x10008), need, None) == WORKSPACE


def test_partition_lengths_for_every_block_size(lib):
    f = lib.pkv_decode_partition_tokens
    # default: 512 tokens, at most 64 blocks of the wave's list (blocks of
    # fewer than 16 tokens: 512 tokens, the list kept in windows of 64)
    assert f(4, 8, 8, 64, 1024, 1, 0) == 512
    assert f(4, 8, 8, 64, 1024, 8, 0) == 512
    assert f(4, 8, 8, 64, 1024, 64, 0) == 512
    assert f(4, 8, 8, 64, 3, 8, 0) == 24          # a short table: one partition
    # requested: blocks below 16 tokens need a multiple of 16
    assert f(4, 8, 8, 64, 1024, 8, 24) == 0
    assert f(4, 8, 8, 64, 1024, 8, 32) == 32
    assert f(4, 8, 8, 64, 1024, 1, 48) == 48
    assert f(4, 8, 8, 64, 1024, 1, 80) == 80      # 80 blocks of one token: two windows
    assert f(4, 8, 8, 64, 1024, 1, 512) == 512
    assert f(4, 8, 8, 64, 1024, 1, 528) == 0      # beyond 512 tokens
    assert f(4, 8, 8, 64, 1024, 8, 576) == 0      # beyond 64 blocks
    assert f(4, 8, 8, 64, 1024, 64, 4096) == 4096


def test_unpartitioned_multi_token_kernel_support(lib):
    # PKV_PARTITION_NONE needs bf16 or FP8 pools with blocks of 16 tokens or more
    assert mq(lib, P=-1, d=desc(dtype=0)) == UNSUPPORTED
    assert mq(lib, P=-1, d=desc(dtype=1, B=8)) == UNSUPPORTED
    # and no workspace, whatever the table length
    assert lib.paged_multi_token_attention(FAKE, None, 8, 2, FAKE, FAKE, FAKE, FAKE, 4, 8, 4096,
                                           ctypes.byref(desc(dtype=1)), 0.125, FAKE, None, 0, -1, None, 0,
                                           None) == INVALID


def test_output_type_flag_is_checked(lib):
    d = desc(dtype=1)
    d.out_f32 = 2
    assert attn(lib, d=d) == INVALID
    d.out_f32 = 1
    assert attn(lib, d=d, S=0) == OK


def step_static(lib, *, S=4, Hq=8, M=4, d=None, P=0):
    d = d or desc()
    return lib.paged_decode_step_static(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, S, Hq, M, ctypes.byref(d), 0.125,
                                        FAKE, None, P, None)


def test_static_step_checks_arguments_before_anything_else(lib):
    # sizes whose workspace exceeds the library's device array, bad sizes and
    # descriptors: rejected on the host, nothing touched
    big = desc(nb=1, hkv=8, B=32, hs=128, dtype=1)
    assert pkv.step_workspace_bytes(512, 64, 8, 128, 4096, 32) > pkv.STATIC_SCRATCH_BYTES
    assert step_static(lib, S=512, Hq=64, M=4096, d=big) == WORKSPACE
    assert step_static(lib, S=-1) == INVALID
    assert step_static(lib, d=desc(hs=96)) == UNSUPPORTED
    assert step_static(lib, S=0) == OK


def test_static_scratch_size_matches_the_header():
    text = open(HEADER).read()
    m = re.search(r"#define PKV_STATIC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == pkv.STATIC_SCRATCH_BYTES


def validate(lib, *, bt=FAKE, sl=FAKE, S=4, M=4, slots=None, T=0, rc=None, d=None, report=FAKE):
    d = d or desc()
    return lib.pkv_validate(bt, sl, S, M, slots, T, rc, ctypes.byref(d), report, None)


def test_validate_rejects_bad_arguments(lib):
    # every check happens on the host, before the report is touched
    assert validate(lib, report=None) == INVALID
    assert validate(lib, report=ctypes.c_void_p(0x10004)) == INVALID  # report not 8-byte aligned
    assert validate(lib, S=-1) == INVALID
    assert validate(lib, M=0) == INVALID
    assert validate(lib, bt=None) == INVALID
    assert validate(lib, sl=None) == INVALID
    assert validate(lib, slots=FAKE, T=-1) == INVALID
    assert validate(lib, d=desc(hs=96)) == UNSUPPORTED
    assert validate(lib, d=desc(nb=0)) == INVALID


def test_validate_report_layout():
    # the binding's field list follows the header's struct, in order
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    body = re.search(r"typedef struct \{([^}]*)\} pkv_validate_report;", text).group(1)
    assert tuple(re.findall(r"int64_t\s+(\w+);", body)) == pkv.VALIDATE_FIELDS
