"""Resource checks on the built gfx950 code objects (CPU only, no GPU).

The kernels keep their accumulators and load rings in registers and LDS; a
kernel that the compiler had to give private (scratch) memory runs several
times slower, with correct results, so no parity test notices it. This test
reads the AMDGPU metadata note of every code object in the library and
fails on any kernel with a private segment, a vector-register spill or a
dynamic stack. It reads only what this repository builds.
"""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

from latency_decode_gemm_amd import _capi

LLVM_BIN = "/opt/rocm/llvm/bin"
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"


def _tool(name):
    path = os.path.join(LLVM_BIN, name)
    if not os.access(path, os.X_OK):
        pytest.skip(f"{path} not available")
    return path


def _kernels():
    """(name, fields) for every kernel of every gfx950 code object in the
    library's .hip_fatbin section (one offload bundle per translation unit)."""
    lib = _capi.LIB_PATH
    if not os.path.exists(lib):
        pytest.skip("library not built")
    objcopy, bundler, readelf = (_tool("llvm-objcopy"), _tool("clang-offload-bundler"),
                                 _tool("llvm-readelf"))
    out = []
    tmp = tempfile.mkdtemp(prefix="skg_co_")
    try:
        fat = os.path.join(tmp, "fatbin")
        subprocess.run([objcopy, "--dump-section", f".hip_fatbin={fat}", lib,
                        os.path.join(tmp, "copy.so")], check=True)
        data = open(fat, "rb").read()
        starts = [m.start() for m in re.finditer(re.escape(MAGIC), data)]
        assert starts, "no offload bundle in the library"
        for i, s in enumerate(starts):
            end = starts[i + 1] if i + 1 < len(starts) else len(data)
            part, co = os.path.join(tmp, f"b{i}"), os.path.join(tmp, f"b{i}.co")
            with open(part, "wb") as f:
                f.write(data[s:end])
            subprocess.run([bundler, "--unbundle", "--type=o", f"--targets={TARGET}",
                            f"--input={part}", f"--output={co}"], check=True)
            notes = subprocess.run([readelf, "--notes", co], check=True,
                                   capture_output=True, text=True).stdout
            for block in notes.split("\n  - .agpr_count:")[1:]:
                name = re.search(r"^\s+\.name:\s+(\S+)", block, re.M).group(1)
                fields = dict(re.findall(r"^\s+\.(\w+):\s+(\S+)$", block, re.M))
                out.append((name, fields))
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return out


def test_no_kernel_uses_scratch_or_spills():
    kernels = _kernels()
    names = [n for n, _ in kernels]
    # every kernel family of the library is in the code objects
    for family in ("skg_valu_kernel", "skg_mfma_kernel", "skg_mfma_ring_kernel",
                   "skg_splitk_reduce_kernel", "skg_small_k_kernel"):
        assert any(family in n for n in names), family
    # (SGPR spills go to lanes of a VGPR, not to memory, and are allowed:
    # a private segment of 0 shows that none reached scratch.)
    bad = [(n, f.get("private_segment_fixed_size"), f.get("vgpr_spill_count"),
            f.get("uses_dynamic_stack"))
           for n, f in kernels
           if f.get("private_segment_fixed_size") != "0" or f.get("vgpr_spill_count") != "0"
           or f.get("uses_dynamic_stack") != "false"]
    assert not bad, f"{len(bad)} of {len(kernels)} kernels use scratch: {bad[:5]}"


def test_kernels_fit_register_and_lds_limits():
    """Every kernel's VGPRs (arch + accumulation registers) fit the 512 a
    wave can hold, and its LDS fits the 160 KB of a CU."""
    for name, f in _kernels():
        assert int(f["vgpr_count"]) + int(f.get("agpr_count", "0")) <= 512, name
        assert int(f["group_segment_fixed_size"]) <= 160 * 1024, name
