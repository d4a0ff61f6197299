"""Benchmark of the MoBA causal prefill on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload h32]

One step is one whole ``moba_prefill_fwd`` call (block mean-pool, gate and
causal top-k, query lists, block attention, LSE merge) on inputs already
resident in HBM, including the workspace taken from the library's stream-ordered
pool. Untimed calls for --settle-ms of wall time (the shader clock ramps up
over the first ~40 ms of load) and then W untimed warm-up calls precede the K
timed ones, which run with nothing else on the stream. Prints one JSON
line with the effective TFLOP/s (only the attended, causal (query, key) pairs
of the selected blocks count, 4*D FLOPs each), the fraction of the bf16 MFMA
peak, per-stage device times from HIP events the library records on its
stream, the roofline of the dominant kernel (the past-block attention launch,
timed by HIP events the library records around it in K further calls), and the
fp64 oracle timed on the host on a sample of query rows.

A ``dense`` object times the same inputs with top_k = n (every block kept:
causal attention, counted as N(N+1)/2 pairs per head). A ``varlen`` object
times the same tokens as 8 packed sequences of N/8 tokens. A ``pooling``
object times the prefill with max and weighted block pooling. A ``backward``
object times ``moba_prefill_bwd`` (dQ, dK, dV for a seeded upstream gradient)
on the same inputs, effective TFLOP/s counted as 2.5x the forward's
attended-pair work. A ``decode`` object times ``moba_decode_fwd`` for the
newest token of the same K/V cache (block means kept from the prefill, as a
generation loop keeps them): once gated with the workload's top-k and once
with top-k above the block count (full attention over the whole cache).
Decode reads 4*D bytes of keys and values per attended key and head, so it is
priced against HBM.

A ``configs`` object times the other workloads of the same family (the long
contexts n128k and m1, the one-head c32k and the fp32 tiny case): whole-call
time, effective TFLOP/s and % of peak, the past-block kernel's launch time, and
for the long ones the oracle on a seeded sample of query rows with a labelled
full-size extrapolation.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoBA prefill effective TFLOP/s + % bf16 MFMA peak at 32K/B512/top-3, 1 GPU"
PEAK_BF16_TFLOPS = 2500.0     # MI355X published dense bf16 MFMA peak
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attention_h32_traffic.json")
ATTN_SRC = os.path.join(ROOT, "block_sparse_long_gating_amd", "csrc", "attn.hip")


def effective_pairs(N: int, B: int, topk: int) -> int:
    """Attended (query, key) pairs of one head: every row of block j sees
    min(topk-1, j) past blocks in full and its own block up to itself."""
    n = N // B
    return sum(B * B * min(topk - 1, j) + B * (B + 1) // 2 for j in range(n))


def past_pairs(N: int, B: int, topk: int) -> int:
    """Attended (query, key) pairs of one head in past (non-own) blocks: the
    work of the past-block attention kernel."""
    n = N // B
    return sum(B * B * min(topk - 1, j) for j in range(n))


def stage_rooflines(w, stage_ms: dict) -> dict:
    """Per-stage bounds of the prefill from the stage times: bytes each stage
    must move in this design over its time, against the HBM peak (the pool,
    the gate and the own-block pass with the merge fused in are bound by HBM;
    the past-block pass is the MFMA-bound kernel of `roofline`)."""
    N, H, D, B, k = w.N, w.H, w.D, w.block_size, w.topk
    n = N // B
    lmax = min(k - 1, n - 1)
    list_entries = H * sum(B * min(k - 1, j) for j in range(n))
    tensor = N * H * D * 2                     # one bf16 [N][H][D] tensor
    parts = {
        # K read once; fp32 means and their 3-way bf16 split written.
        "pool": ("pool", tensor + H * n * D * (4 + 6),
                 "K read once; K-bar fp32 and its bf16 split written"),
        # Q read once; the selection rows, in-tile ranks and per-tile counts written.
        "gate": ("gate", tensor + H * N * (k + lmax) * 4 + H * n * -(-N // 128) * 4,
                 "Q read once; selection rows, in-tile ranks and per-tile counts written"),
        # Own block: Q, K, V read once; past partial rows (bf16) and their lse read
        # back; out and lse written.
        "attn_own_merge": ("attn_own", 3 * tensor + list_entries * (2 * D + 4) + tensor + H * N * 4,
                           "Q, K, V read once; past partials (bf16 rows + lse) read back; out and lse written"),
    }
    out = {}
    for name, (stage, nbytes, what) in parts.items():
        t = stage_ms.get(stage, 0.0) + (stage_ms.get("merge", 0.0) if name == "attn_own_merge" else 0.0)
        gbs = nbytes / (t * 1e-3) / 1e9 if t > 0 else 0.0
        out[name] = {"bound": "hbm", "bytes": nbytes, "us": 1e3 * t, "achieved": gbs, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS, "bytes_counted": what}
    out["timing"] = ("stage times from HIP events the library records at its stage boundaries "
                     "(launch gaps included)")
    return out


def row_pairs(rows: np.ndarray, B: int, topk: int) -> int:
    j = rows // B
    return int(np.sum(np.minimum(topk - 1, j) * B + rows % B + 1))


def device_info():
    import torch
    p = torch.cuda.get_device_properties(0)
    info = {"name": p.name, "cus": p.multi_processor_count, "arch": getattr(p, "gcnArchName", "")}
    try:
        import ctypes
        hip = ctypes.CDLL("libamdhip64.so")
        clk = ctypes.c_int()
        # hipDeviceAttributeClockRate (kHz)
        if hip.hipDeviceGetAttribute(ctypes.byref(clk), 5, 0) == 0 and clk.value > 0:
            info["clock_mhz"] = clk.value / 1000.0
    except OSError:
        pass
    return info


def code_sha256(path: str) -> str:
    """sha256 of a C++/HIP source with its comments and blank lines removed, so
    that it changes with the code and not with the comments."""
    with open(path) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = [re.sub(r"//.*$", "", line).rstrip() for line in text.splitlines()]
    return hashlib.sha256("\n".join(line for line in lines if line).encode()).hexdigest()


def traffic_for(workload: str):
    """HBM bytes per launch of the past-block attention kernel from the
    committed rocprofv3 counter summary, if it was taken on this workload with
    the current kernel code (else None)."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        t = json.load(f)
    if t.get("attn_code_sha256") != code_sha256(ATTN_SRC) or t.get("workload") != workload:
        return None
    return t.get("bytes_per_launch")


def decode_bench(moba, w, qd, kd, vd, steps: int):
    """Decode step for the token at position N - 1 of the cache: gated with the
    workload's top-k and as full attention (top-k = number of blocks)."""
    import torch
    q_new = qd[w.N - 1].contiguous()
    kbar = moba.block_mean_keys(kd, w.block_size)
    out = torch.empty_like(q_new)
    lse = torch.empty((w.H,), dtype=torch.float32, device=qd.device)
    n_blocks = (w.N + w.block_size - 1) // w.block_size
    j = (w.N - 1) // w.block_size
    res = {}
    for name, topk in (("moba", w.topk), ("full", n_blocks)):
        kept = min(topk, j + 1)
        keys = (kept - 1) * w.block_size + (w.N - j * w.block_size)
        nbytes = w.H * keys * 4 * w.D
        for _ in range(5):
            moba.decode(q_new, kd, vd, w.block_size, topk, kbar=kbar, out=out, lse=lse)
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        for _ in range(steps):
            moba.decode(q_new, kd, vd, w.block_size, topk, kbar=kbar, out=out, lse=lse)
        stop.record()
        torch.cuda.synchronize()
        us = 1e3 * start.elapsed_time(stop) / steps
        res[name] = {"top_k": topk, "kept_blocks": kept, "attended_keys": keys, "us_per_step": us,
                     "kv_gbytes": nbytes / 1e9, "achieved_gbs": nbytes / (us * 1e-6) / 1e9,
                     "frac_hbm": nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS}
    res["speedup_vs_full"] = res["full"]["us_per_step"] / res["moba"]["us_per_step"]
    res["timing"] = ("back-to-back calls through the Python binding between two HIP events on the stream; "
                     "host launch overhead is included where it exceeds the kernels' time")
    return res


def backward_bench(moba, w, qd, kd, vd, out, lse, steps: int, warmup: int):
    """moba_prefill_bwd on the same workload (upstream gradient: seeded N(0, 1))."""
    import torch
    from block_sparse_long_gating_amd import synth
    do = torch.from_numpy(synth.bf16_bits(synth.make_grad(w.N, w.H, w.D, seed=[402, 9]))).view(torch.bfloat16)
    do = do.to(qd.device)
    dq, dk, dv = torch.empty_like(qd), torch.empty_like(qd), torch.empty_like(qd)
    for _ in range(warmup):
        moba.prefill_backward(qd, kd, vd, out, lse, do, w.block_size, w.topk, dq=dq, dk=dk, dv=dv)
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(steps):
        moba.prefill_backward(qd, kd, vd, out, lse, do, w.block_size, w.topk, dq=dq, dk=dk, dv=dv)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    # FlashAttention convention: the backward of an attended pair is 2.5x its
    # forward work (S, dP, dV, dQ, dK: five D-long products, 10 D FLOPs).
    flops = 10.0 * w.D * effective_pairs(w.N, w.block_size, w.topk) * w.H
    return {"ms_per_step": ms, "effective_gflop": flops / 1e9, "effective_tflops": flops / (ms * 1e-3) / 1e12,
            "pct_peak": 100.0 * flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "includes": "block mean-pool, gate, query lists (recomputed), delta, dK/dV, dQ"}


def pooling_bench(moba, w, qd, kd, vd, steps: int):
    """The prefill with max and with weighted block pooling (weights: seeded
    uniform [0, 1) per head and token); only the pool stage differs."""
    import torch
    wts = torch.from_numpy(np.random.default_rng([403, 0]).uniform(0.0, 1.0, (w.H, w.N)).astype(np.float32))
    wts = wts.to(qd.device)
    flops = 4.0 * w.D * effective_pairs(w.N, w.block_size, w.topk) * w.H
    res = {}
    for pooling in ("max", "weighted"):
        args = (qd, kd, vd, w.block_size, w.topk, pooling, wts if pooling == "weighted" else None)
        for _ in range(3):
            moba.prefill_pooled(*args)
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        for _ in range(steps):
            moba.prefill_pooled(*args)
        stop.record()
        torch.cuda.synchronize()
        ms = start.elapsed_time(stop) / steps
        res[pooling] = {"ms_per_step": ms, "effective_tflops": flops / (ms * 1e-3) / 1e12}
    return res


def dense_bench(moba, w, qd, kd, vd, steps: int):
    """top_k = n on the same inputs: every block kept, i.e. causal attention
    over the whole sequence (the dense path; hybrid full-attention layers)."""
    import torch
    n = w.N // w.block_size
    for _ in range(2):
        moba.prefill(qd, kd, vd, w.block_size, n)
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(steps):
        moba.prefill(qd, kd, vd, w.block_size, n)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    flops = 4.0 * w.D * w.H * w.N * (w.N + 1) / 2
    return {"top_k": n, "ms_per_step": ms, "causal_gflop": flops / 1e9,
            "effective_tflops": flops / (ms * 1e-3) / 1e12,
            "pct_peak": 100.0 * flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}


def varlen_bench(moba, w, qd, kd, vd, steps: int, nseq: int = 8):
    """The same tokens as ``nseq`` packed sequences of N / nseq tokens each."""
    import torch
    L = w.N // nseq
    cu = [i * L for i in range(nseq + 1)]
    for _ in range(2):
        moba.prefill_varlen(qd, kd, vd, cu, w.block_size, w.topk)
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(steps):
        moba.prefill_varlen(qd, kd, vd, cu, w.block_size, w.topk)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    flops = 4.0 * w.D * w.H * nseq * effective_pairs(L, w.block_size, w.topk)
    return {"sequences": nseq, "tokens_each": L, "ms_per_step": ms, "effective_gflop": flops / 1e9,
            "effective_tflops": flops / (ms * 1e-3) / 1e12}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_flops(w, rows: np.ndarray) -> float:
    """FLOPs the oracle itself spends on ``rows`` (all heads) with its
    per-block evaluation: every chosen block's B logits twice (row maxima,
    then exponentials) and its B values once, 6 D B per chosen block and row,
    plus the gate's scores against all n block means, 2 D n per row."""
    j = rows // w.block_size
    kept = np.minimum(w.topk, j + 1)
    n = w.N // w.block_size
    return float(w.H * np.sum(6.0 * w.D * w.block_size * kept + 2.0 * w.D * n))


def sample_parity(w, q, k, rows, out, lse, sel, gpu_out_rows, gpu_lse_rows, gpu_sel_rows):
    """GPU results against the oracle's on sampled rows: outputs compared on
    the (row, head) pairs whose selection equals the oracle's; differing
    selections checked for the near-tie exemption (both denominators)."""
    from tests.parity import compare_selection
    same = np.all(gpu_sel_rows == sel, axis=2)                   # [H, R]
    d_out = np.max(np.abs(gpu_out_rows.astype(np.float64) - out), axis=2).T   # [H, R]
    d_lse = np.abs(gpu_lse_rows - lse)                           # [H, R]
    cmp = compare_selection(gpu_sel_rows, sel, q, k, w.block_size, w.topk, rows=rows)
    return {
        "rows": int(rows.shape[0]),
        "pairs_same_selection": int(same.sum()),
        "pairs_other_selection": int((~same).sum()),
        "other_selection_near_tie": cmp["exempt"],
        "other_selection_near_tie_rowmax": cmp["exempt_rowmax"],
        "other_selection_not_tie": len(cmp["bad"]),
        "max_abs_out": float(np.max(d_out[same])) if same.any() else None,
        "max_abs_lse": float(np.max(d_lse[same])) if same.any() else None,
    }


def cpu_baseline(w, q, k, v, gpu_out, gpu_lse, gpu_sel, target_s: float):
    """The fp64 oracle as it stands, on a seeded sample of query rows; the
    GPU outputs are compared with it on the (row, head) pairs whose block
    selection matches the oracle's (the others differ at near-ties of the
    gate scores, where either choice is correct)."""
    import threadpoolctl

    from block_sparse_long_gating_amd import synth
    from oracle import moba_ref

    cores = len(os.sched_getaffinity(0))
    blas = threadpoolctl.threadpool_info()
    threads = max([b.get("num_threads", 1) for b in blas] + [1])
    R = min(1024, w.N)
    while True:
        rows = synth.sample_rows(w.N, R, 2000 + R)
        t0 = time.perf_counter()
        out, lse, sel = moba_ref(q, k, v, w.block_size, w.topk, rows=rows)
        dt = time.perf_counter() - t0
        # Part of the oracle's cost does not grow with the rows (the block
        # means), so the estimate from a small sample undershoots: take
        # another, larger sample until it lasts at least 0.6 target_s.
        if dt >= 0.6 * target_s or R >= w.N:
            break
        R = min(w.N, int(R * max(2.0, target_s / max(dt, 1e-3))))
    flops = 4.0 * w.D * w.H * row_pairs(rows, w.block_size, w.topk)
    full = R >= w.N
    res = {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{R} seeded query rows x {w.H} heads of the {w.name} workload "
                  f"(gate over all blocks + fp64 softmax over the attended keys); {dt:.2f} s; "
                  f"{cores} cores visible, BLAS threads {threads}",
        "cpu_model": cpu_model(),
        "cores_visible": cores,
        "seconds": dt,
        "rows": int(R),
        "rows_per_s": R * w.H / dt,
        "effective_gflop": flops / 1e9,
        "oracle_gflop": oracle_flops(w, rows) / 1e9,
        "oracle_gflops_rate": oracle_flops(w, rows) / dt / 1e9,
        "full_call_s": dt if full else None,
        "full_call_s_extrapolated": None if full else dt * w.N / R,
    }
    res_parity = sample_parity(w, q, k, rows, out, lse, sel, gpu_out[rows], gpu_lse[:, rows], gpu_sel[:, rows, :])
    return res, res_parity


def settle(call, ms: float, min_calls: int = 3) -> int:
    """Untimed calls until `ms` of wall time have passed (at least min_calls):
    brings the shader clock to its loaded level. Returns the number of calls."""
    import torch
    torch.cuda.synchronize()
    t_end = time.perf_counter() + ms * 1e-3
    calls = 0
    while calls < min_calls or time.perf_counter() < t_end:
        call()
        calls += 1
        if calls % 10 == 0 or calls == min_calls:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return calls


def configs_bench(moba, names, steps: int, cpu_rows: int, with_cpu: bool, settle_ms: float):
    """The whole prefill call on the other workloads (their own inputs),
    with the past-block kernel's launch time, and the oracle on a seeded row
    sample of the long ones (GPU parity on the same rows)."""
    import torch

    from block_sparse_long_gating_amd import synth
    res = {}
    for name in names:
        w, q, k, v = synth.make_workload(name)
        dev = torch.device("cuda:0")
        if w.dtype == "bf16":
            qd, kd, vd = (torch.from_numpy(synth.bf16_bits(x)).view(torch.bfloat16).to(dev) for x in (q, k, v))
        else:
            qd, kd, vd = (torch.from_numpy(x).to(dev) for x in (q, k, v))
        out = torch.empty_like(qd)
        lse = torch.empty((w.H, w.N), dtype=torch.float32, device=dev)
        nsteps = steps if effective_pairs(w.N, w.block_size, w.topk) * w.H < 10 ** 10 else max(3, steps // 4)
        settle(lambda: moba.prefill(qd, kd, vd, w.block_size, w.topk, out=out, lse=lse), settle_ms)
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        for _ in range(nsteps):
            moba.prefill(qd, kd, vd, w.block_size, w.topk, out=out, lse=lse)
        stop.record()
        torch.cuda.synchronize()
        ms = start.elapsed_time(stop) / nsteps
        flops = 4.0 * w.D * w.H * effective_pairs(w.N, w.block_size, w.topk)
        r = {"N": w.N, "H": w.H, "D": w.D, "block_size": w.block_size, "top_k": w.topk, "dtype": w.dtype,
             "steps": nsteps, "ms_per_step": ms, "effective_gflop": flops / 1e9,
             "effective_tflops": flops / (ms * 1e-3) / 1e12,
             "pct_peak": 100.0 * flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
        if w.dtype == "bf16":
            events = [moba.StageEvents(stages=("attn_past",)) for _ in range(nsteps)]
            for i in range(nsteps):
                moba.prefill(qd, kd, vd, w.block_size, w.topk, out=out, lse=lse, events=events[i])
            torch.cuda.synchronize()
            for e in events:
                e.accumulate()
            past_ms = sum(e.totals["attn_past"] for e in events) / nsteps
            for e in events:
                e.close()
            pf = 4.0 * w.D * w.H * past_pairs(w.N, w.block_size, w.topk)
            r["past_kernel"] = {"launch_us": 1e3 * past_ms, "gflop": pf / 1e9,
                                "tflops": pf / (past_ms * 1e-3) / 1e12 if past_ms > 0 else None,
                                "frac": pf / (past_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS if past_ms > 0 else None}
        print(f"[bench] {name}: {ms:.3f} ms/step, {r['effective_tflops']:.1f} effective TFLOP/s "
              f"({r['pct_peak']:.1f}% of peak)", file=sys.stderr, flush=True)
        if with_cpu and name in ("n128k", "m1"):
            from oracle import moba_ref
            rows = synth.sample_rows(w.N, cpu_rows, synth.SAMPLE_SEED[name])
            t0 = time.perf_counter()
            o_out, o_lse, o_sel = moba_ref(q, k, v, w.block_size, w.topk, rows=rows)
            dt = time.perf_counter() - t0
            of = oracle_flops(w, rows)
            ef = 4.0 * w.D * w.H * row_pairs(rows, w.block_size, w.topk)
            r["cpu_oracle"] = {
                "kind": "oracle", "rows": int(rows.shape[0]), "heads": w.H, "seconds": dt,
                "rows_per_s": rows.shape[0] * w.H / dt, "effective_tflops": ef / dt / 1e12,
                "oracle_gflop": of / 1e9, "cpu_model": cpu_model(),
                "full_call_s_extrapolated": dt * w.N / rows.shape[0],
                "note": "sampled rows; the full-size time is extrapolated linearly in the row count",
            }
            sel = moba.gate_topk(qd, kd, w.block_size, w.topk).cpu().numpy()[:, rows, :]
            r["parity_sample"] = sample_parity(w, q, k, rows, o_out, o_lse, o_sel,
                                               out.float().cpu().numpy()[rows], lse.cpu().numpy()[:, rows], sel)
        res[name] = r
        del qd, kd, vd, out, lse, q, k, v
        torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="h32")
    ap.add_argument("--cpu-baseline", choices=("on", "off"), default="on")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--dense", choices=("on", "off"), default="on",
                    help="also time the prefill with every block kept (causal attention)")
    ap.add_argument("--varlen", choices=("on", "off"), default="on",
                    help="also time the same tokens as 8 packed sequences")
    ap.add_argument("--pooling", choices=("on", "off"), default="on",
                    help="also time the prefill with max and weighted block pooling")
    ap.add_argument("--backward", choices=("on", "off"), default="on",
                    help="also time the backward pass on the same workload")
    ap.add_argument("--decode", choices=("on", "off"), default="on",
                    help="also time the decode step on the same cache")
    ap.add_argument("--configs", default="n128k,m1,c32k,tiny",
                    help="other workloads to time after the headline one (comma list; 'none' for none)")
    ap.add_argument("--config-cpu-rows", type=int, default=1024,
                    help="oracle rows sampled per long workload for its CPU time and parity")
    ap.add_argument("--settle-ms", type=float, default=150.0,
                    help="before the warm-up calls, keep the GPU busy with prefill calls for this long (ms of wall "
                         "time): the shader clock ramps up over the first ~40 ms of load")
    ap.add_argument("--per-call-ms", type=int, default=0,
                    help="before the warm-up, time this many single calls with HIP events (prints them)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="after timing, run plain device copies of this size (HBM counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by head with no communication between GPUs)", file=sys.stderr)
        sys.exit(2)

    import torch

    import block_sparse_long_gating_amd as moba
    from block_sparse_long_gating_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    moba.load_library()
    w, q, k, v = synth.make_workload(args.workload)
    if w.dtype != "bf16":
        print("bench.py times the bf16 path", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")

    def up(x):
        return torch.from_numpy(synth.bf16_bits(x)).view(torch.bfloat16).to(dev)

    qd, kd, vd = up(q), up(k), up(v)
    out = torch.empty_like(qd)
    lse = torch.empty((w.H, w.N), dtype=torch.float32, device=dev)
    print(f"[bench] workload {w.name}: {w.description}", file=sys.stderr, flush=True)

    if args.per_call_ms > 0:
        # Per-call device times from the first call on (warm-up behaviour).
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.per_call_ms)]
        for a, b in evs:
            a.record()
            moba.prefill(qd, kd, vd, w.block_size, w.topk, out=out, lse=lse)
            b.record()
        torch.cuda.synchronize()
        times = [a.elapsed_time(b) for a, b in evs]
        print("[bench] per-call ms: " + " ".join(f"{t:.3f}" for t in times), file=sys.stderr, flush=True)

    # Clock settle: the shader clock rises from ~1.8 to ~2.3 GHz over the first
    # ~40 ms of continuous load while every kernel's cycle count stays the same
    # (per-dispatch GRBM_GUI_ACTIVE against the dispatch time), so the first
    # calls of a process measure the power state, not the code. Prefill calls
    # run until settle_ms of wall time have passed; they are reported.
    settle_calls = 0
    if args.settle_ms > 0:
        settle_calls = settle(lambda: moba.prefill(qd, kd, vd, w.block_size, w.topk, out=out, lse=lse),
                              args.settle_ms, min_calls=1)

    for _ in range(args.warmup):
        moba.prefill(qd, kd, vd, w.block_size, w.topk, out=out, lse=lse)
    torch.cuda.synchronize()

    # Timed region: K whole calls and nothing else on the stream.
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        moba.prefill(qd, kd, vd, w.block_size, w.topk, out=out, lse=lse)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps

    # Launch time of the dominant kernel: K more calls with the two boundaries
    # around the past-block attention launch recorded by the library on its
    # stream (kept out of the loop above: each recorded event costs the stream
    # a few us).
    events = [moba.StageEvents(stages=("attn_past",)) for _ in range(args.steps)]
    start.record()
    for i in range(args.steps):
        moba.prefill(qd, kd, vd, w.block_size, w.topk, out=out, lse=lse, events=events[i])
    stop.record()
    torch.cuda.synchronize()
    ms_with_events = start.elapsed_time(stop) / args.steps
    for e in events:
        e.accumulate()
    past_ms = sum(e.totals["attn_past"] for e in events) / args.steps
    for e in events:
        e.close()

    # Stage breakdown (informative), from a few more calls with every boundary recorded.
    stage_steps = max(3, min(args.steps, 10))
    events = [moba.StageEvents() for _ in range(stage_steps)]
    for i in range(stage_steps):
        moba.prefill(qd, kd, vd, w.block_size, w.topk, out=out, lse=lse, events=events[i])
    torch.cuda.synchronize()
    for e in events:
        e.accumulate()
    stage_ms = {s: sum(e.totals[s] for e in events) / stage_steps for s in moba.STAGES}
    for e in events:
        e.close()
    print(f"[bench] {args.steps} steps, {ms:.3f} ms/step, stages (us): "
          + ", ".join(f"{s} {1e3 * t:.1f}" for s, t in stage_ms.items()), file=sys.stderr, flush=True)

    if args.calibrate_copy_mib > 0:
        nbytes = args.calibrate_copy_mib << 20
        src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    pairs = effective_pairs(w.N, w.block_size, w.topk) * w.H
    flops = 4.0 * w.D * pairs
    tflops = flops / (ms * 1e-3) / 1e12
    # Dominant kernel: the past-block attention launch; its algorithmic work is
    # the attended pairs in past blocks, 4 D FLOPs each.
    past_flops = 4.0 * w.D * past_pairs(w.N, w.block_size, w.topk) * w.H
    past_tflops = past_flops / (past_ms * 1e-3) / 1e12 if past_ms > 0 else 0.0
    info = device_info()

    result = {
        "metric": METRIC,
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_settle": {"calls": settle_calls, "ms": args.settle_ms,
                         "why": "untimed prefill calls before the warm-up: the shader clock ramps from ~1.8 to "
                                "~2.3 GHz over the first ~40 ms of load (kernel cycle counts constant)"},
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "N": w.N, "H": w.H, "D": w.D, "block_size": w.block_size,
                   "top_k": w.topk, "batch": 1, "inputs": w.description},
        "pct_peak": 100.0 * tflops / PEAK_BF16_TFLOPS,
        "effective_gflop": flops / 1e9,
        "stages_us": {s: 1e3 * t for s, t in stage_ms.items()},
        "roofline": {
            "bound": "mfma",
            "kernel": "attn_mfma_kernel<128, past blocks> (block attention over the query lists)",
            "achieved": past_tflops,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": past_tflops / PEAK_BF16_TFLOPS,
            "traffic": traffic_for(w.name),
            "algorithmic_gflop_per_launch": past_flops / 1e9,
            "launch_us": 1e3 * past_ms,
            "launch_timing": f"{args.steps} further calls with HIP events around this launch "
                             f"({ms_with_events:.3f} ms per call with the events)",
        },
        "stage_rooflines": stage_rooflines(w, stage_ms),
        "device": info,
    }

    if args.dense == "on":
        result["dense"] = dense_bench(moba, w, qd, kd, vd, max(3, args.steps // 4))
        dn = result["dense"]
        print(f"[bench] dense (top-k = n): {dn['ms_per_step']:.3f} ms, {dn['effective_tflops']:.1f} TFLOP/s",
              file=sys.stderr, flush=True)

    if args.varlen == "on":
        result["varlen"] = varlen_bench(moba, w, qd, kd, vd, max(5, args.steps // 2))
        vl = result["varlen"]
        print(f"[bench] varlen ({vl['sequences']} x {vl['tokens_each']}): {vl['ms_per_step']:.3f} ms, "
              f"{vl['effective_tflops']:.1f} effective TFLOP/s", file=sys.stderr, flush=True)

    if args.pooling == "on":
        result["pooling"] = pooling_bench(moba, w, qd, kd, vd, max(5, args.steps // 2))
        pl = result["pooling"]
        print(f"[bench] pooled prefill: max {pl['max']['ms_per_step']:.3f} ms, "
              f"weighted {pl['weighted']['ms_per_step']:.3f} ms", file=sys.stderr, flush=True)

    if args.backward == "on":
        result["backward"] = backward_bench(moba, w, qd, kd, vd, out, lse, args.steps, args.warmup)
        bw = result["backward"]
        print(f"[bench] backward: {bw['ms_per_step']:.3f} ms/step, {bw['effective_tflops']:.1f} effective TFLOP/s",
              file=sys.stderr, flush=True)

    if args.decode == "on":
        result["decode"] = decode_bench(moba, w, qd, kd, vd, max(50, 10 * args.steps))
        d = result["decode"]
        print(f"[bench] decode: gated {d['moba']['us_per_step']:.1f} us, full {d['full']['us_per_step']:.1f} us "
              f"({d['full']['achieved_gbs']:.0f} GB/s)", file=sys.stderr, flush=True)

    if args.cpu_baseline == "on":
        torch.cuda.synchronize()
        got_out = out.float().cpu().numpy()
        got_lse = lse.cpu().numpy()
        got_sel = moba.gate_topk(qd, kd, w.block_size, w.topk).cpu().numpy()
        cb, parity = cpu_baseline(w, q, k, v, got_out, got_lse, got_sel, args.cpu_seconds)
        result["cpu_baseline"] = cb
        result["parity_sample"] = parity
    else:
        result["cpu_baseline"] = None

    names = [x for x in args.configs.split(",") if x and x != "none" and x != w.name]
    if names:
        del qd, kd, vd, out, lse
        torch.cuda.empty_cache()
        result["configs"] = configs_bench(moba, names, args.steps, args.config_cpu_rows, args.cpu_baseline == "on",
                                          args.settle_ms)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
