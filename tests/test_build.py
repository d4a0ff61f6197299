"""CPU check of the compiled kernels: no private (scratch) memory.

(The backward and decode kernels keep their accumulators and operands in
registers; a spill there would not change results either, only speed.)

The attention and gate kernels count their own outstanding vector-memory
operations and wait on exact counts. A register spilled to scratch and
reloaded inside the tile loop makes the compiler wait for every outstanding
operation instead (it cannot see the inline-asm loads), which drains the load
ring on every tile without changing any result, so only this check sees it.
"""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_sparse_long_gating_amd", "csrc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-S", "--cuda-device-only"]


def kernel_metadata(src, tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    out = tmp_path / (os.path.basename(src) + ".s")
    subprocess.run([hipcc, *FLAGS, "-o", str(out), src], check=True, capture_output=True)
    meta = {}
    name = None
    for line in out.read_text().splitlines():
        m = re.match(r"\s+\.name:\s+(\S+)", line)
        if m:
            name = m.group(1)
            meta[name] = {}
            continue
        m = re.match(r"\s+\.(private_segment_fixed_size|vgpr_spill_count|sgpr_spill_count|vgpr_count):\s+(\d+)", line)
        if m and name is not None:
            meta[name][m.group(1)] = int(m.group(2))
    return meta


@pytest.mark.parametrize("src,pattern", [("attn.hip", "attn_mfma_kernel"), ("gate.hip", "gate_mfma_kernel"),
                                         ("bwd.hip", "bwd_"), ("decode.hip", "decode_")])
def test_mfma_kernels_use_no_scratch(src, pattern, tmp_path):
    meta = kernel_metadata(os.path.join(CSRC, src), tmp_path)
    kernels = {k: v for k, v in meta.items() if pattern in k}
    assert kernels, f"no {pattern} kernels found in {src}"
    for k, v in kernels.items():
        assert v.get("private_segment_fixed_size") == 0, (k, v)
        assert v.get("vgpr_spill_count") == 0, (k, v)
