"""CPU: register and scratch budgets of the gfx950 kernels in the built
libqmoe.so, read from the code objects' metadata (no GPU needed).

A kernel that spills to scratch memory turns its register reloads into
memory round trips inside the pipelined K loops; a grouped-GEMM change that
pushed the stage-1 kernels past their register budget once cost the a8w4
stage 1 a quarter of its speed with the outputs unchanged, so no parity test
could see it.  This test fails on any kernel that uses scratch, except the
listed variants that always have (and that no rule of the library picks).
"""
import os
import re
import shutil
import struct
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "quantized_mixture_experts_moe_amd", "libqmoe.so")
READELF = "/opt/rocm/llvm/bin/llvm-readelf"
BUNDLE_MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"

# Mangled-name fragments of the kernels allowed a little scratch: the a8w4
# 128-row tiles of 4 waves (stage 1 canonical layout, stage 2 row-major),
# reachable only through QMOE_TILE s1w=4 / s2w=4, 12 bytes each.
ALLOWED_SCRATCH = {
    "moe_gemm_kernelILi2ELi1ELi128ELb0ELi2ELi4ELb1ELi4ELb0E": 12,
    "moe_gemm_kernelILi2ELi2ELi128ELb1ELi2ELi4ELb0ELi4ELb0E": 12,
}


def _code_objects(path):
    """The gfx950 code objects of the library's offload bundles."""
    out = subprocess.run([READELF, "-S", "-W", path], capture_output=True, text=True,
                         check=True).stdout
    off = size = None
    for line in out.splitlines():
        parts = line.split()
        if ".hip_fatbin" in parts:
            i = parts.index(".hip_fatbin")
            off, size = int(parts[i + 3], 16), int(parts[i + 4], 16)
    assert off is not None, "no .hip_fatbin section"
    with open(path, "rb") as f:
        f.seek(off)
        data = f.read(size)
    objs, pos = [], 0
    while True:
        j = data.find(BUNDLE_MAGIC, pos)
        if j < 0:
            break
        (n,) = struct.unpack_from("<Q", data, j + len(BUNDLE_MAGIC))
        q = j + len(BUNDLE_MAGIC) + 8
        for _ in range(n):
            eo, es, il = struct.unpack_from("<QQQ", data, q)
            q += 24
            ident = data[q:q + il].decode()
            q += il
            if ident == TARGET and es > 0:
                objs.append(data[j + eo:j + eo + es])
        pos = j + len(BUNDLE_MAGIC)
    return objs


def _kernels(obj_bytes):
    """(name, fields) of every kernel in one code object's metadata note."""
    with tempfile.NamedTemporaryFile(suffix=".co") as f:
        f.write(obj_bytes)
        f.flush()
        notes = subprocess.run([READELF, "--notes", f.name], capture_output=True, text=True,
                               check=True).stdout
    out = []
    for block in notes.split("\n      - ")[1:]:
        m = re.search(r"\.name:\s+(\S+)", block)
        if not m or m.group(1).endswith(".kd"):
            continue
        fields = {}
        for key in ("vgpr_count", "agpr_count", "private_segment_fixed_size",
                    "vgpr_spill_count", "sgpr_spill_count"):
            v = re.search(r"\." + key + r":\s+(\d+)", block)
            if v:
                fields[key] = int(v.group(1))
        out.append((m.group(1), fields))
    return out


@pytest.fixture(scope="module")
def kernels():
    if not os.path.exists(LIB):
        pytest.skip("libqmoe.so is not built")
    if not (os.path.exists(READELF) or shutil.which("llvm-readelf")):
        pytest.skip("llvm-readelf is not available")
    ks = []
    for obj in _code_objects(LIB):
        ks += _kernels(obj)
    return ks


def test_every_source_contributes_kernels(kernels):
    names = " ".join(n for n, _ in kernels)
    for frag in ("moe_gemm_kernel", "moe_stage2_resident", "decode_kernel", "route_kernel",
                 "combine_kernel", "requant_kernel", "align_count_kernel", "prepack_codes_kernel"):
        assert frag in names, frag
    assert len(kernels) > 200


def test_no_kernel_uses_scratch(kernels):
    bad = []
    for name, f in kernels:
        scratch = f.get("private_segment_fixed_size", 0)
        allowed = next((v for k, v in ALLOWED_SCRATCH.items() if k in name), 0)
        if scratch > allowed:
            bad.append((name, scratch, f.get("vgpr_spill_count"), f.get("sgpr_spill_count")))
    assert not bad, f"kernels using scratch: {bad[:8]}"
