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
# Near-tie exemption for the top-k (the tie clause of the parity bar: a
# selection may differ only where the gating scores are within 1e-4 relative).
# A differing selection is accepted only if, score for score (both sets sorted),
# |g_a - g_b| <= TIE_REL * max(|g_a|, |g_b|), with the oracle's fp32 scores.
# The looser count, with the row's largest past-block |score| as the
# denominator, is reported beside it.
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


def near_tie(g, a, b, rel=TIE_REL, lo=0, j=None):
    """Whether the past-block sets ``a`` (oracle) and ``b`` (GPU) of one row
    are a near-tie under the fp32 scores ``g`` of that row: returns (pairwise,
    row-max), the first with the pair denominator max(|g_a|, |g_b|), the second
    with the row's largest |score| over its candidate blocks lo..j-1."""
    sa = np.sort(np.asarray(g, np.float64)[list(a)])[::-1]
    sb = np.sort(np.asarray(g, np.float64)[list(b)])[::-1]
    if sa.shape != sb.shape:
        return False, False
    gap = np.abs(sa - sb)
    pair = bool(np.all(gap <= rel * np.maximum(np.abs(sa), np.abs(sb))))
    hi = j if j is not None else len(g)
    rowmax = float(np.max(np.abs(np.asarray(g, np.float64)[lo:hi]))) if hi > lo else 0.0
    return pair, bool(np.all(gap <= rel * rowmax))


def compare_selection(gpu_sel, ref_sel, q, k, B, topk, rows=None, rel=TIE_REL, pooling="mean", weights=None,
                      scores=None):
    """Compare [H, R, topk] selections row by row.

    A row may differ from the oracle's only if (1) its -1 padding sits in
    exactly the oracle's slots, (2) the gate had a choice to make (more past
    blocks than the k - 1 kept ones; a row with j < topk must match exactly),
    (3) it is a valid selection (ascending, distinct, block j last, every
    other entry a past block) and (4) the differing past blocks are a near-tie
    (``near_tie``). Returns a dict: rows compared, mismatched rows, exempt
    rows under the pairwise rule and under the row-max rule, and the
    (h, t, oracle, gpu) of rows failing each rule ("bad" is the pairwise one).
    ``scores`` ([H, R, n] fp32) skips recomputing the oracle's gate scores.
    """
    gpu_sel = np.asarray(gpu_sel)
    ref_sel = np.asarray(ref_sel)
    H, R, _ = ref_sel.shape
    rows = np.arange(R) if rows is None else np.asarray(rows)
    diff = np.nonzero((gpu_sel != ref_sel).any(axis=-1))
    result = {"rows": int(H * R), "mismatch": int(diff[0].size), "exempt": 0, "exempt_rowmax": 0,
              "bad": [], "bad_rowmax": []}
    if diff[0].size == 0:
        return result
    if scores is None:
        sub_rows = np.unique(rows[diff[1]])
        sc = oracle_scores(q, k, B, sub_rows, pooling, weights)
        where = {int(t): i for i, t in enumerate(sub_rows)}
    else:
        sc = np.asarray(scores)
        where = {int(t): i for i, t in enumerate(rows)}
    for h, r in zip(*diff):
        t = int(rows[r])
        j = t // B
        gs, rs = gpu_sel[h, r], ref_sel[h, r]
        entry = (int(h), t, [int(x) for x in rs], [int(x) for x in gs])
        pad_ok = bool(np.array_equal(gs == -1, rs == -1))
        ranked = j >= topk                     # j past blocks compete for k - 1 slots
        b = [int(x) for x in gs if x >= 0]
        valid = (b == sorted(set(b)) and len(b) == topk and b[-1] == j and b[0] >= 0
                 and all(x >= -1 for x in gs))
        pair = rowmax = False
        if pad_ok and ranked and valid:
            a = [int(x) for x in rs if x >= 0 and x != j]
            pair, rowmax = near_tie(sc[h, where[t]], a, b[:-1], rel, 0, j)
        if pair:
            result["exempt"] += 1
        else:
            result["bad"].append(entry)
        if rowmax:
            result["exempt_rowmax"] += 1
        else:
            result["bad_rowmax"].append(entry)
    return result


def max_abs(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64)))) if np.size(a) else 0.0
