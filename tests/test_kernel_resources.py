"""Register budgets of the built kernels, read from the gfx950 code objects
inside libpkv.so (the AMDGPU metadata notes the compiler wrote): no kernel
spills to scratch memory, and the decode attention variants of the benchmark
shapes keep the waves per SIMD their loads are sized for.  CPU only: it reads
the library file, nothing runs."""
import os
import re
import shutil
import struct
import subprocess

import pytest
import yaml

import paged_kv_cache_35_amd as pkv

LLVM = "/opt/rocm/llvm/bin"
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"


def tool(name):
    path = os.path.join(LLVM, name)
    return path if os.path.exists(path) else shutil.which(name)


@pytest.fixture(scope="module")
def kernels(tmp_path_factory):
    if not os.path.exists(pkv.LIB_PATH):
        pytest.fail("libpkv.so is not built (run __graft_entry__.build())")
    objcopy, readelf = tool("llvm-objcopy"), tool("llvm-readelf")
    if not objcopy or not readelf:
        pytest.skip("LLVM tools of the ROCm toolchain not found")
    d = tmp_path_factory.mktemp("co")
    fatbin = d / "fatbin"
    subprocess.run([objcopy, f"--dump-section=.hip_fatbin={fatbin}", pkv.LIB_PATH, str(d / "lib")], check=True)
    data = fatbin.read_bytes()
    # the linked section holds one offload bundle per source file, back to back
    out, pos, n = {}, 0, 0
    while (i := data.find(MAGIC, pos)) >= 0:
        count = struct.unpack_from("<Q", data, i + 24)[0]
        off = i + 32
        for _ in range(count):
            o, size, tl = struct.unpack_from("<QQQ", data, off)
            triple = data[off + 24:off + 24 + tl].decode()
            off += 24 + tl
            if "gfx950" in triple and size:
                co = d / f"co{n}.elf"
                co.write_bytes(data[i + o:i + o + size])
                n += 1
                notes = subprocess.run([readelf, "--notes", str(co)], capture_output=True, text=True,
                                       check=True).stdout
                text = notes[notes.index("---"):]
                for k in yaml.safe_load(text[:text.index("\n...")])["amdhsa.kernels"]:
                    out[k[".name"]] = k
        pos = i + len(MAGIC)
    assert n >= 7, "one gfx950 code object per source file expected"
    return out


def waves_per_simd(k):
    """Waves of this kernel one SIMD holds by its registers: 512 per lane,
    allocated in granules of 8.  On gfx950 .vgpr_count is the unified count:
    the architected registers (rounded up to 4) plus the accumulation
    registers, which .agpr_count repeats."""
    assert k[".vgpr_count"] >= k[".agpr_count"]
    regs = -(-k[".vgpr_count"] // 8) * 8
    return min(8, 512 // regs)


def test_no_kernel_spills_to_scratch(kernels):
    spilled = {n: k[".private_segment_fixed_size"] for n, k in kernels.items() if k[".private_segment_fixed_size"]}
    assert not spilled, f"kernels using scratch memory: {spilled}"


@pytest.mark.parametrize("elem,hs,bs,f8,mq,waves", [
    ("DF16b", 128, 16, 0, 0, 3), ("DF16b", 128, 32, 0, 0, 2), ("DF16b", 128, 64, 0, 0, 2),
    ("DF16b", 128, 16, 1, 0, 3), ("DF16b", 128, 32, 1, 0, 2), ("DF16b", 128, 64, 1, 0, 2),
    ("DF16b", 128, 16, 0, 1, 3), ("DF16b", 128, 16, 1, 1, 3), ("DF16b", 128, 32, 1, 1, 2),
])
def test_decode_attention_occupancy(kernels, elem, hs, bs, f8, mq, waves):
    # decode (mq 0) and multi-token (mq 1) instantiations of the partition kernel
    pat = re.compile(rf"paged_decode_partition_kernelI{elem}Li{hs}ELi{bs}ELi4ELb{f8}ELb{mq}E")
    found = [k for n, k in kernels.items() if pat.search(n)]
    assert len(found) == 1
    got = waves_per_simd(found[0])
    assert got >= waves, f"{found[0]['.vgpr_count']} + {found[0]['.agpr_count']} registers: {got} waves per SIMD"
