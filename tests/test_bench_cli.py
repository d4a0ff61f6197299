"""CPU checks of bench.py's command line (no GPU is touched)."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT, env=env,
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = run_bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""          # no JSON line


def test_launch_with_several_ranks_is_refused():
    r = run_bench("--gpus", "1", env_extra={"WORLD_SIZE": "4"})
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def test_help_names_the_contract_flags():
    r = run_bench("--help")
    assert r.returncode == 0
    for flag in ("--gpus", "--steps", "--warmup", "--workload"):
        assert flag in r.stdout


def test_stage_rooflines_count_the_stage_bytes():
    """Per-stage HBM bounds on the tiny shape (N=2048, H=1, D=64, block 256,
    top-3: 8 blocks), bytes counted by hand."""
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench_module", os.path.join(ROOT, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    from block_sparse_long_gating_amd import synth
    w = synth.WORKLOADS["tiny"]
    r = bench.stage_rooflines(w, {"pool": 0.001, "gate": 0.002, "attn_own": 0.004, "merge": 0.0})
    tensor = 2048 * 64 * 2
    assert r["pool"]["bytes"] == tensor + 8 * 64 * 10
    # selection rows (3) + in-tile ranks (2) per query, 16 per-tile counts per block
    assert r["gate"]["bytes"] == tensor + 2048 * 5 * 4 + 8 * 16 * 4
    # list entries: 256 * (0 + 1 + 2 * 6) = 3328 rows of 2 * 64 + 4 bytes
    assert r["attn_own_merge"]["bytes"] == 4 * tensor + 3328 * 132 + 2048 * 4
    assert abs(r["pool"]["achieved"] - r["pool"]["bytes"] / 1e-6 / 1e9) < 1e-6
    assert abs(r["pool"]["frac"] * 8000.0 - r["pool"]["achieved"]) < 1e-6
