"""Resource use of the built gfx950 kernels, read from the code-object metadata of the library's own objects.

Every kernel must run without per-lane scratch memory (no register spills, no private segment): a kernel
that spills needs the HIP runtime to provide scratch backing at launch, which the library's callers (graph
capture, callers that cannot allocate) do not expect, and spilled GEMM loops run at a fraction of their rate.
The 256x256 GEMM shapes run two waves per SIMD, so each of their waves must fit in 256 VGPRs.
"""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "fp8_fine_grained_amax_amd", "csrc")
LLVM = "/opt/rocm/llvm/bin"
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"


def _sources():
    import importlib.util
    spec = importlib.util.spec_from_file_location("fg_build", os.path.join(ROOT, "fp8_fine_grained_amax_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod.SOURCES


def _kernel_metadata(obj):
    """[(kernel name, {field: int})] from the gfx950 code object bundled in one host object."""
    with tempfile.TemporaryDirectory() as d:
        fatbin, co = os.path.join(d, "fatbin"), os.path.join(d, "co.o")
        subprocess.run([f"{LLVM}/llvm-objcopy", f"--dump-section=.hip_fatbin={fatbin}", obj, os.path.join(d, "x")],
                       check=True, capture_output=True)
        subprocess.run([f"{LLVM}/clang-offload-bundler", "--type=o", f"--targets={TARGET}", f"--input={fatbin}",
                        f"--output={co}", "--unbundle"], check=True, capture_output=True)
        notes = subprocess.run([f"{LLVM}/llvm-readelf", "--notes", co], check=True, capture_output=True,
                               text=True).stdout
    out = []
    # one top-level list entry per kernel ("  - ." at the start of a line); the argument lists nested in
    # each entry are indented further
    for block in re.split(r"^  - \.", notes, flags=re.M)[1:]:
        name = re.search(r"\.name:\s+(\S+)", block)
        if not name or not name.group(1).startswith("_Z"):
            continue
        fields = {k: int(v) for k, v in re.findall(r"\.(\w+):\s+(\d+)\s*$", block, re.M)}
        out.append((name.group(1), fields))
    return out


@pytest.fixture(scope="module")
def kernels():
    if not all(os.path.exists(os.path.join(LLVM, t)) for t in ("llvm-objcopy", "clang-offload-bundler", "llvm-readelf")):
        pytest.skip("LLVM object tools not found under /opt/rocm/llvm/bin")
    objs = [os.path.join(CSRC, s.replace(".hip", ".o")) for s in _sources()]
    missing = [o for o in objs if not os.path.exists(o)]
    if missing:
        pytest.skip("library objects not built (run __graft_entry__.build()): " + ", ".join(map(os.path.basename, missing)))
    found = {}
    for o in objs:
        if os.path.basename(o) == "api.o":
            continue                         # host-side argument checks only
        for name, f in _kernel_metadata(o):
            found[name] = f
    return found


def test_every_source_has_kernels(kernels):
    assert any("fg_gemm_kernel" in n for n in kernels)
    assert any("fg_quant_x_both_w_kernel" in n for n in kernels)
    assert len(kernels) >= 30


def test_no_scratch_no_spills(kernels):
    bad = {n: (f.get("private_segment_fixed_size"), f.get("vgpr_spill_count"), f.get("sgpr_spill_count"))
           for n, f in kernels.items()
           if f.get("private_segment_fixed_size", 0) or f.get("vgpr_spill_count", 0) or f.get("sgpr_spill_count", 0)}
    assert not bad, f"kernels with scratch (private bytes, vgpr spills, sgpr spills): {bad}"


def test_gemm_register_budget(kernels):
    # TileCfg<2, 4, ...> is the 8-wave 256x256 shape and fg_gemm_wide_kernel the 8-wave 256x288 one (2 waves
    # per SIMD, 256 VGPRs each); TileCfg<4, 3, ...> the 12-wave 256x192 shape (3 waves per SIMD, 168 VGPRs
    # each, rounded to the granule)
    assert any("fg_gemm_wide_kernel" in n for n in kernels)
    for n, f in kernels.items():
        if "fg_gemm_kernel" not in n and "fg_gemm_wide_kernel" not in n:
            continue
        limit = 256 if ("TileCfgILi2ELi4E" in n or "fg_gemm_wide_kernel" in n) else 168
        assert f["vgpr_count"] <= limit, (n, f["vgpr_count"])
