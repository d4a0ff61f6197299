"""CPU checks of the compiled kernels: no private (scratch) memory, and the
dK/dV loop's row loads kept in flight across the tile's products.

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


def loop_bodies(asm, kernel):
    """Instructions of each loop of `kernel` in layout order, keyed by loop header."""
    start = asm.index(kernel + ":")
    body = asm[start:asm.index(".Lfunc_end", start)].splitlines()
    loops, cur = {}, None
    for line in body:
        m = re.match(r"^(\.LBB\d+_\d+):.*(?:Loop Header|in Loop: Header=(\S+))", line)
        if m:
            cur = m.group(1) if "Loop Header" in line else ".L" + m.group(2)
            loops.setdefault(cur, [])
            continue
        if re.match(r"^(\.LBB|; %bb)", line):
            if "in Loop" not in line and "Loop Header" not in line:
                cur = None
            continue
        t = line.strip()
        if cur is not None and t and not t.startswith(";"):
            loops[cur].append(t)
    return loops


def test_dkdv_row_loads_stay_in_flight_during_the_tile(tmp_path):
    """In the dK/dV pipeline the next tile's Q/dO rows are loaded at the start of
    a step and committed to LDS at its end; a full vmcnt wait before the step's
    first product means the compiler waits for the loads it has just issued
    (it did when a list entry was widened right after its load), and the rows'
    latency is no longer hidden behind the tile. Only speed depends on it."""
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    out = tmp_path / "bwd.s"
    subprocess.run([hipcc, *FLAGS, "-o", str(out), os.path.join(CSRC, "bwd.hip")], check=True, capture_output=True)
    asm = out.read_text()
    kernel = next(m.group(1) for m in re.finditer(r"^(_Z\S*bwd_dkdv_kernelILi128E\S*):", asm, re.M))
    checked = 0
    for header, ins in loop_bodies(asm, kernel).items():
        ops = [x.split()[0] for x in ins]
        if "global_load_dwordx4" not in ops or not any(o.startswith("v_mfma") for o in ops):
            continue
        first_load = ops.index("global_load_dwordx4")
        first_mfma = next(i for i in range(first_load, len(ops)) if ops[i].startswith("v_mfma"))
        full_waits = [i for i in range(first_load, len(ins)) if ins[i].startswith("s_waitcnt vmcnt(0)")]
        assert not full_waits or full_waits[0] > first_mfma, (header, full_waits[:1], first_mfma)
        checked += 1
    assert checked >= 1
