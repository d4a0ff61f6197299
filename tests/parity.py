"""Helpers shared by the GPU parity tests and the benchmark's parity leg:
device upload, selection comparison with the near-tie exemption, and
output comparison against the oracle."""

from __future__ import annotations

import sys

import numpy as np

from block_sparse_long_gating_amd import synth

# Tolerances. Outputs: max abs error (bf16 with fp32 accumulation / fp32 inputs).
OUT_TOL = {"bf16": 2e-2, "fp32": 1e-4}
# lse (natural log): not fixed by the pages; bf16 rounding of the logits' inputs
# is exact, so the error is that of fp32 accumulation plus exp2/log2.
LSE_TOL = {"bf16": 1e-2, "fp32": 1e-5}
# Near-tie exemption for the top-k: a selection that differs from the oracle's
# is accepted only if, score for score, the chosen past blocks' fp32 scores
# agree within this fraction of the row's largest past-block |score|.
TIE_REL = 1e-4


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(x: np.ndarray, dtype: str, device="cuda"):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(synth.bf16_bits(x)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(device)


def oracle_scores(q, k, B, rows, pooling="mean", weights=None):
    """fp32 gate scores [H, R, n] from the oracle."""
    from oracle import gate_scores, pooled_keys_fp32
    kbar32 = pooled_keys_fp32(k, B, pooling, weights)
    H = q.shape[1]
    return np.stack([gate_scores(q[rows, h, :], kbar32[h]) for h in range(H)])


def compare_selection(gpu_sel, ref_sel, q, k, B, topk, rows=None, rel=TIE_REL, pooling="mean", weights=None):
    """Compare [H, R, topk] selections. Returns a dict with the number of
    mismatched rows, how many of them are exempt near-ties, and the (h, r) of
    any that are not."""
    gpu_sel = np.asarray(gpu_sel)
    ref_sel = np.asarray(ref_sel)
    H, R, _ = ref_sel.shape
    rows = np.arange(R) if rows is None else np.asarray(rows)
    diff = np.nonzero((gpu_sel != ref_sel).any(axis=-1))
    result = {"rows": int(H * R), "mismatch": int(diff[0].size), "exempt": 0, "bad": []}
    if diff[0].size == 0:
        return result
    sub_rows = np.unique(rows[diff[1]])
    sc = oracle_scores(q, k, B, sub_rows, pooling, weights)
    where = {int(t): i for i, t in enumerate(sub_rows)}
    for h, r in zip(*diff):
        t = int(rows[r])
        j = t // B
        g = sc[h, where[t]].astype(np.float64)
        a = [int(x) for x in ref_sel[h, r] if x >= 0 and x != j]
        b = [int(x) for x in gpu_sel[h, r] if x >= 0]
        ok = (len(b) == len(a) + 1 and j in b and b == sorted(set(b)) and max(b) == j
              and all(x >= -1 for x in gpu_sel[h, r]))
        if ok:
            bp = [x for x in b if x != j]
            tol = rel * float(np.max(np.abs(g[:j]))) if j > 0 else 0.0
            sa = np.sort(g[a])[::-1]
            sb = np.sort(g[bp])[::-1]
            ok = bool(np.all(np.abs(sa - sb) <= tol))
        if ok:
            result["exempt"] += 1
        else:
            result["bad"].append((int(h), t, a, b))
    return result


def max_abs(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64)))) if np.size(a) else 0.0
