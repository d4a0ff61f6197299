"""Pins that tie the fp64 oracle to facts fixed outside of it.

Every ``pin_*`` function takes an oracle module ``m`` (the real one, or a copy
with a planted mistake) and raises ``AssertionError`` when ``m`` disagrees with
what the pages or the mathematics fix:

* numbers the pages print (tests/golden/pages_pins.json),
* brute force on tiny inputs through independent routes (exhaustive subset
  search for the top-k, torch's masked SDPA for the attention),
* special cases that reduce to a library routine (top_k >= n is full causal
  attention; top_k = 1 is block-diagonal causal attention),
* closed forms and invariants.
"""

from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_pins.json")


def golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _rand(N, H, D, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((N, H, D)).astype(np.float32) * np.float32(scale)
    k = rng.standard_normal((N, H, D)).astype(np.float32) * np.float32(scale)
    v = rng.standard_normal((N, H, D)).astype(np.float32)
    return q, k, v


def _t64(x):
    return torch.from_numpy(np.asarray(x, np.float64))


# ---------------------------------------------------------------------------
# independent brute force
# ---------------------------------------------------------------------------

def brute_selection(q, k, B, topk, kbar=None):
    """Top-k by exhaustive subset search, computed with torch (not numpy).

    For each query the chosen past blocks are the (k-1)-subset of eligible
    blocks with the largest score sum; among equal sums the lexicographically
    smallest index tuple wins (that is the lower-index tie rule). The gate
    scores are the exact dot products with the fp32-rounded block means,
    rounded to fp32.
    """
    N, H, D = q.shape
    n = N // B
    if kbar is None:
        kt = _t64(k).reshape(n, B, H, D)
        kbar = kt.mean(dim=1).to(torch.float32).to(torch.float64)     # [n, H, D]
    sel = np.full((H, N, topk), -1, np.int64)
    for h in range(H):
        sc = (_t64(q[:, h, :]) @ kbar[:, h, :].T).to(torch.float32).to(torch.float64).numpy()
        for t in range(N):
            j = t // B
            if j + 1 <= topk:
                chosen = list(range(j + 1))
            else:
                best, best_sum = None, -math.inf
                for comb in itertools.combinations(range(j), topk - 1):
                    s = sum(sc[t, i] for i in comb)
                    if s > best_sum:
                        best, best_sum = comb, s
                chosen = sorted(list(best) + [j])
            sel[h, t, :len(chosen)] = chosen
    return sel


def brute_attention(q, k, v, B, sel):
    """Masked attention through torch SDPA in fp64, mask built token by token."""
    N, H, D = q.shape
    out = np.zeros((N, H, D))
    lse = np.zeros((H, N))
    for h in range(H):
        mask = torch.zeros((N, N), dtype=torch.bool)
        for t in range(N):
            for s in range(t + 1):
                if (s // B) in set(int(x) for x in sel[h, t] if x >= 0):
                    mask[t, s] = True
        qh, kh, vh = _t64(q[:, h]), _t64(k[:, h]), _t64(v[:, h])
        o = torch.nn.functional.scaled_dot_product_attention(
            qh[None], kh[None], vh[None], attn_mask=mask[None])
        out[:, h] = o[0].numpy()
        logits = (qh @ kh.T) / math.sqrt(D)
        lse[h] = torch.logsumexp(logits.masked_fill(~mask, -math.inf), dim=-1).numpy()
    return out, lse


# ---------------------------------------------------------------------------
# pins
# ---------------------------------------------------------------------------

TINY_CASES = [  # (N, H, D, B, topk, seed)
    (16, 2, 4, 2, 3, 11),
    (32, 1, 4, 4, 2, 12),
    (48, 2, 4, 4, 4, 13),
    (64, 1, 4, 8, 3, 14),
    (40, 1, 4, 8, 1, 15),
    (24, 2, 4, 2, 5, 16),
]


def pin_bruteforce_tiny(m):
    for N, H, D, B, topk, seed in TINY_CASES:
        q, k, v = _rand(N, H, D, seed)
        out, lse, sel = m.moba_ref(q, k, v, B, topk)
        bsel = brute_selection(q, k, B, topk)
        assert np.array_equal(sel, bsel), f"selection differs from exhaustive search at {N, B, topk}"
        bout, blse = brute_attention(q, k, v, B, bsel)
        assert np.allclose(out, bout, rtol=0, atol=1e-12), f"output differs from masked SDPA at {N, B, topk}"
        assert np.allclose(lse, blse, rtol=0, atol=1e-12), f"lse differs from masked logsumexp at {N, B, topk}"


def pin_chunked_loops(m):
    """The oracle's chunk loops against the brute-force routes, with chunks so
    small that every call runs several of them and a ragged last one: the gate
    over row chunks of 7 (select_blocks), and the dense attention over row
    chunks of 5 inside each query block (moba_ref's max_rows_chunk)."""
    for N, H, D, B, topk, seed in TINY_CASES:
        q, k, v = _rand(N, H, D, seed)
        bsel = brute_selection(q, k, B, topk)
        sel, _ = m.select_blocks(q, k, B, topk, chunk=7)
        assert np.array_equal(sel, bsel), f"chunked selection differs from exhaustive search at {N, B, topk}"
        rows = np.arange(3, N, 2)          # a row subset: chunk boundaries fall between chosen rows
        sel_r, _ = m.select_blocks(q, k, B, topk, rows=rows, chunk=7)
        assert np.array_equal(sel_r, bsel[:, rows]), f"chunked row-subset selection differs at {N, B, topk}"
        bout, blse = brute_attention(q, k, v, B, bsel)
        out, lse, _ = m.moba_ref(q, k, v, B, topk, method="dense", max_rows_chunk=5)
        assert np.allclose(out, bout, rtol=0, atol=1e-12), f"chunked dense output differs at {N, B, topk}"
        assert np.allclose(lse, blse, rtol=0, atol=1e-12), f"chunked dense lse differs at {N, B, topk}"
        out_r, lse_r, _ = m.moba_ref(q, k, v, B, topk, rows=rows, method="dense", max_rows_chunk=3)
        assert np.allclose(out_r, bout[rows], rtol=0, atol=1e-12), f"chunked row-subset output differs at {N, B}"
        assert np.allclose(lse_r, blse[:, rows], rtol=0, atol=1e-12), f"chunked row-subset lse differs at {N, B}"


def pin_full_causal(m):
    """top_k >= n selects every past block: plain causal attention."""
    for N, H, D, B, seed in [(64, 2, 8, 8, 21), (96, 1, 16, 16, 22)]:
        q, k, v = _rand(N, H, D, seed)
        n = N // B
        for topk in (n, n + 3):
            out, lse, sel = m.moba_ref(q, k, v, B, topk)
            for h in range(H):
                qh, kh, vh = _t64(q[:, h]), _t64(k[:, h]), _t64(v[:, h])
                ref = torch.nn.functional.scaled_dot_product_attention(qh[None], kh[None], vh[None], is_causal=True)[0]
                assert np.allclose(out[:, h], ref.numpy(), atol=1e-12, rtol=0)
                logits = (qh @ kh.T) / math.sqrt(D)
                causal = torch.ones(N, N, dtype=torch.bool).tril()
                rl = torch.logsumexp(logits.masked_fill(~causal, -math.inf), -1)
                assert np.allclose(lse[h], rl.numpy(), atol=1e-12, rtol=0)


def pin_block_diagonal(m):
    """top_k = 1 keeps only the own block: block-diagonal causal attention."""
    N, H, D, B = 64, 2, 8, 16
    q, k, v = _rand(N, H, D, 31)
    out, lse, sel = m.moba_ref(q, k, v, B, 1)
    for h in range(H):
        for j in range(N // B):
            s = slice(j * B, (j + 1) * B)
            ref = torch.nn.functional.scaled_dot_product_attention(
                _t64(q[s, h])[None], _t64(k[s, h])[None], _t64(v[s, h])[None], is_causal=True)[0]
            assert np.allclose(out[s, h], ref.numpy(), atol=1e-12, rtol=0)
    assert np.all(sel[:, :, 0] == (np.arange(N) // B)[None, :])


def pin_first_token(m):
    N, H, D, B = 32, 2, 8, 8
    q, k, v = _rand(N, H, D, 41)
    out, lse, _ = m.moba_ref(q, k, v, B, 3)
    for h in range(H):
        assert np.array_equal(out[0, h], v[0, h].astype(np.float64))
        exact = float(np.dot(q[0, h].astype(np.float64), k[0, h].astype(np.float64))) / math.sqrt(D)
        assert abs(lse[h, 0] - exact) < 1e-13


def pin_constant_v(m):
    N, H, D, B = 48, 1, 8, 8
    q, k, _ = _rand(N, H, D, 51)
    v = np.broadcast_to(np.linspace(-2, 2, D, dtype=np.float32), (N, H, D)).copy()
    out, _, _ = m.moba_ref(q, k, v, B, 3)
    assert np.allclose(out, v.astype(np.float64), atol=1e-13, rtol=0)


def pin_zero_query(m):
    """q = 0: every score ties, the tie rule alone decides, attention is uniform."""
    N, H, D, B, topk = 64, 1, 8, 8, 3
    _, k, v = _rand(N, H, D, 61)
    q = np.zeros((N, H, D), np.float32)
    out, lse, sel = m.moba_ref(q, k, v, B, topk)
    for t in range(N):
        j = t // B
        expect = list(range(j + 1)) if j + 1 <= topk else list(range(topk - 1)) + [j]
        assert list(sel[0, t, :len(expect)]) == expect, (t, sel[0, t])
        keys = [s for s in range(t + 1) if (s // B) in expect]
        assert np.allclose(out[t, 0], v[keys, 0].astype(np.float64).mean(0), atol=1e-13)
        assert abs(lse[0, t] - math.log(len(keys))) < 1e-13


def pin_invariants(m):
    N, H, D, B = 256, 3, 16, 16
    q, k, v = _rand(N, H, D, 71)
    for topk in (1, 2, 3, 5, 16, 20):
        sel, _ = m.select_blocks(q, k, B, topk)
        for h in range(H):
            for t in range(N):
                j = t // B
                row = [int(x) for x in sel[h, t] if x >= 0]
                assert len(row) == min(topk, j + 1)
                assert row == sorted(set(row))
                assert j in row and max(row) == j and min(row) >= 0
                assert all(x == -1 for x in sel[h, t, len(row):])


def pin_pages_worked_example(m):
    g = golden()["worked_example"]
    N, B, topk, D = g["N"], g["block_size"], g["top_k"], g["head_dim"]
    rng = np.random.default_rng(81)
    k = rng.standard_normal((N, 1, D)).astype(np.float32)
    q = rng.standard_normal((N, 1, D)).astype(np.float32)
    rows = np.array([N - 1])
    sel, _ = m.select_blocks(q, k, B, topk, rows=rows)
    chosen = [int(x) for x in sel[0, 0] if x >= 0]
    assert len(chosen) == g["blocks_selected"]
    tokens = len(m.attended_keys(sel[0, 0], N - 1, B))
    assert tokens == g["tokens_attended"]
    assert round(100 * (1 - tokens / N), 2) == g["sparsity_percent_2dp"]
    assert round(100 * m.sparsity(N, B, topk), 2) == g["sparsity_percent_2dp"]


def pin_pages_sparsity_table(m):
    rows = golden()["sparsity_table"]["rows"]
    snippet = golden()["config_snippet"]
    assert m.n_blocks(snippet["context_length"], snippet["block_size"]) == snippet["num_blocks"]
    assert round(100 * m.sparsity(snippet["context_length"], snippet["block_size"], snippet["top_k"]), 1) \
        == snippet["sparsity_percent_1dp"]
    for r in rows:
        N, B, topk = r["N"], r["block_size"], r["top_k"]
        assert round(100 * m.sparsity(N, B, topk), 1) == r["sparsity_percent_1dp"]
        D = 4
        rng = np.random.default_rng(91)
        k = rng.standard_normal((N, 1, D)).astype(np.float32)
        q = rng.standard_normal((N, 1, D)).astype(np.float32)
        last = np.array([N - 1])
        sel, _ = m.select_blocks(q, k, B, topk, rows=last)
        tokens = len(m.attended_keys(sel[0, 0], N - 1, B))
        assert round(100 * (1 - tokens / N), 1) == r["sparsity_percent_1dp"]


def pin_granularity(m):
    for c in golden()["granularity"]["cases"]:
        n, chosen = c["n_blocks"], c["chosen"]
        B, D = 4, 4
        N = n * B
        q, k, _ = _rand(N, 1, D, 101)
        sel, _ = m.select_blocks(q, k, B, chosen, rows=np.array([N - 1]))
        tokens = len(m.attended_keys(sel[0, 0], N - 1, B))
        assert 100 * (1 - tokens / N) == c["sparsity_percent"]
    f = golden()["full_switch"]
    assert m.n_blocks(f["N"], f["block_size"]) == f["n_blocks"]
    assert 100 * m.sparsity(f["N"], f["block_size"], f["top_k"]) == f["sparsity_percent"]


def pin_closed_form_pairs(m):
    for N, B, topk in [(128, 8, 3), (128, 16, 1), (96, 8, 12), (160, 32, 2), (64, 8, 9)]:
        q, k, _ = _rand(N, 1, 4, 111)
        sel, _ = m.select_blocks(q, k, B, topk)
        total = sum(len(m.attended_keys(sel[0, t], t, B)) for t in range(N))
        # closed form, written independently: sum over query blocks j of
        # B*B*min(k-1, j) + B*(B+1)/2
        n = N // B
        direct = sum(B * B * min(topk - 1, j) + B * (B + 1) // 2 for j in range(n))
        assert total == direct == m.attended_pairs_closed_form(N, B, topk)
        assert all(len(m.attended_keys(sel[0, t], t, B)) == m.attended_count(t, B, topk) for t in range(N))


def pin_query_lists_hand_example(m):
    """Lists regrouped by hand from two hand-written selections (N = 8, B = 2,
    top-2): list (h, b) holds the queries t that chose b as a past block."""
    sel = np.array([
        [[0, -1], [0, -1], [0, 1], [0, 1], [1, 2], [0, 2], [2, 3], [0, 3]],
        [[0, -1], [0, -1], [0, 1], [0, 1], [0, 2], [0, 2], [1, 3], [1, 3]],
    ], np.int32)
    offs, qidx = m.query_lists(sel, 2)
    assert offs.tolist() == [0, 4, 5, 6, 6, 10, 12, 12, 12]
    assert qidx.tolist() == [2, 3, 5, 7, 4, 6, 2, 3, 4, 5, 6, 7]
    # topk wider than the eligible blocks: the -1 padding lists nothing.
    offs, qidx = m.query_lists(np.array([[[0, -1, -1], [0, -1, -1], [0, 1, -1], [0, 1, -1]]], np.int32), 2)
    assert offs.tolist() == [0, 2, 2] and qidx.tolist() == [2, 3]


def pin_query_lists_transpose(m):
    """On oracle selections: the lists are the transpose of the selection minus
    the own block (checked through a membership matrix), each list ascending,
    and the total is the closed form H * sum_j B * min(k - 1, j)."""
    for N, H, B, topk in [(96, 2, 8, 3), (128, 3, 16, 20), (64, 1, 8, 1), (160, 2, 32, 2)]:
        q, k, _ = _rand(N, H, 4, 131)
        sel, _ = m.select_blocks(q, k, B, topk)
        offs, qidx = m.query_lists(sel, B)
        n = N // B
        assert offs.shape == (H * n + 1,) and offs[0] == 0
        assert offs[-1] == H * sum(B * min(topk - 1, j) for j in range(n)) == qidx.shape[0]
        member = np.zeros((H, N, n), bool)
        for e in range(H * n):
            lst = qidx[offs[e]:offs[e + 1]]
            assert np.all(np.diff(lst) > 0)
            assert not member[e // n, lst, e % n].any()
            member[e // n, lst, e % n] = True
        for h in range(H):
            for t in range(N):
                want = {int(b) for b in sel[h, t] if 0 <= b < t // B}
                assert set(np.flatnonzero(member[h, t]).tolist()) == want


def pin_lse_merge(m):
    """Merging per-block softmax partials by log-sum-exp equals the oracle's one softmax."""
    N, H, D, B, topk = 96, 2, 8, 8, 4
    q, k, v = _rand(N, H, D, 121)
    out, lse, sel = m.moba_ref(q, k, v, B, topk)
    for h in range(H):
        for t in range(N):
            j = t // B
            parts = []
            for b in sel[h, t]:
                if b < 0:
                    continue
                hi = (b + 1) * B if b < j else t + 1
                ks = torch.from_numpy(k[b * B:hi, h].astype(np.float64))
                vs = torch.from_numpy(v[b * B:hi, h].astype(np.float64))
                lg = ks @ torch.from_numpy(q[t, h].astype(np.float64)) / math.sqrt(D)
                parts.append((torch.logsumexp(lg, 0), torch.softmax(lg, 0) @ vs))
            tot = torch.logsumexp(torch.stack([p[0] for p in parts]), 0)
            merged = sum(torch.exp(p[0] - tot) * p[1] for p in parts)
            assert abs(float(tot) - lse[h, t]) < 1e-12
            assert np.allclose(merged.numpy(), out[t, h], atol=1e-12, rtol=0)


def pin_pooling_linearity(m):
    """Dot with the mean key equals the mean of the per-key dot products."""
    N, H, D, B = 64, 2, 8, 16
    q, k, _ = _rand(N, H, D, 131)
    kbar = m.pooled_keys(k, B)
    assert kbar.shape == (H, N // B, D)
    for h in range(H):
        for t in range(0, N, 7):
            for i in range(N // B):
                per_key = [float(np.dot(q[t, h].astype(np.float64), k[s, h].astype(np.float64)))
                           for s in range(i * B, (i + 1) * B)]
                assert abs(math.fsum(per_key) / B - float(q[t, h].astype(np.float64) @ kbar[h, i])) < 1e-12


def pin_gate_rounding(m):
    """Mean keys and scores are the exact values rounded once to fp32."""
    from fractions import Fraction
    N, H, D, B = 32, 1, 4, 8
    q, k, _ = _rand(N, H, D, 141)
    kb32 = m.pooled_keys_fp32(k, B)
    for i in range(N // B):
        for d in range(D):
            exact = sum(Fraction(float(k[s, 0, d])) for s in range(i * B, (i + 1) * B)) / B
            assert kb32[0, i, d] == np.float32(float(exact))
    sc = m.gate_scores(q[:, 0, :], kb32[0])
    for t in range(N):
        for i in range(N // B):
            exact = sum(Fraction(float(q[t, 0, d])) * Fraction(float(kb32[0, i, d])) for d in range(D))
            assert sc[t, i] == np.float32(float(exact))


def pin_row_mode_matches(m):
    """The three evaluations of the softmax over A(t) agree: dense masked
    logits, per-block logits over the rows that chose the block, and one
    gathered row at a time."""
    for N, H, D, B, topk, seed in [(128, 2, 8, 16, 3, 151), (192, 1, 8, 64, 2, 152), (96, 2, 4, 8, 20, 153)]:
        q, k, v = _rand(N, H, D, seed)
        out, lse, sel = m.moba_ref(q, k, v, B, topk)
        rows = np.unique(np.array([0, 5, B - 1, B, B + 1, N // 2, N - 2, N - 1]))
        for method in ("blocks", "rowwise", "dense"):
            o2, l2, s2 = m.moba_ref(q, k, v, B, topk, rows=rows, method=method)
            assert np.array_equal(s2, sel[:, rows])
            assert np.allclose(o2, out[rows], atol=1e-13, rtol=0), method
            assert np.allclose(l2, lse[:, rows], atol=1e-13, rtol=0), method
        allrows = np.arange(N)
        o3, l3, _ = m.moba_ref(q, k, v, B, topk, rows=allrows, method="blocks")
        assert np.allclose(o3, out, atol=1e-13, rtol=0)
        assert np.allclose(l3, lse, atol=1e-13, rtol=0)


# ---------------------------------------------------------------------------
# decode step (one new token at position N - 1; N need not be a multiple of B)
# ---------------------------------------------------------------------------

def _sdpa_one(qv, kk, vv):
    """Attention of one query over the given keys through torch SDPA (fp64), and its logsumexp."""
    qh, kh, vh = _t64(qv)[None, None], _t64(kk)[None], _t64(vv)[None]
    o = torch.nn.functional.scaled_dot_product_attention(qh, kh, vh)[0, 0].numpy()
    lse = float(torch.logsumexp((kh[0] @ qh[0, 0]) / math.sqrt(qv.shape[-1]), dim=0))
    return o, lse


def pin_decode_full_attention(m):
    """top_k above the number of past blocks: the token attends the whole cache."""
    for N, H, D, B, seed in [(77, 2, 8, 16, 161), (64, 1, 8, 16, 162), (5, 2, 4, 8, 163), (130, 1, 4, 64, 164)]:
        q, k, v = _rand(N, H, D, seed)
        out, lse, sel = m.moba_decode_ref(q[N - 1], k, v, B, (N - 1) // B + 2)
        for h in range(H):
            ro, rl = _sdpa_one(q[N - 1, h], k[:, h], v[:, h])
            assert np.allclose(out[h], ro, atol=1e-12, rtol=0)
            assert abs(lse[h] - rl) < 1e-12
            assert list(sel[h][sel[h] >= 0]) == list(range((N - 1) // B + 1))


def pin_decode_own_block(m):
    """top_k = 1: only the token's own (possibly partial) block, keys jB .. N-1."""
    for N, H, D, B, seed in [(77, 2, 8, 16, 171), (64, 1, 8, 16, 172), (100, 2, 4, 32, 173)]:
        q, k, v = _rand(N, H, D, seed)
        out, lse, sel = m.moba_decode_ref(q[N - 1], k, v, B, 1)
        j0 = ((N - 1) // B) * B
        for h in range(H):
            ro, rl = _sdpa_one(q[N - 1, h], k[j0:, h], v[j0:, h])
            assert np.allclose(out[h], ro, atol=1e-12, rtol=0)
            assert abs(lse[h] - rl) < 1e-12


def pin_decode_first_token(m):
    q, k, v = _rand(1, 2, 8, 181)
    out, lse, sel = m.moba_decode_ref(q[0], k, v, 16, 3)
    for h in range(2):
        assert np.array_equal(out[h], v[0, h].astype(np.float64))
        assert abs(lse[h] - float(np.dot(q[0, h].astype(np.float64), k[0, h].astype(np.float64))) / math.sqrt(8)) < 1e-13
    assert np.array_equal(sel, np.array([[0, -1, -1], [0, -1, -1]]))


def pin_decode_brute_selection(m):
    """The gate of a decode step against exhaustive subset search over the
    complete past blocks (fp32 means and scores through torch)."""
    for N, H, D, B, topk, seed in [(45, 2, 4, 4, 3, 191), (37, 1, 4, 2, 4, 192), (64, 2, 4, 8, 2, 193), (9, 1, 4, 2, 5, 194)]:
        q, k, v = _rand(N, H, D, seed)
        out, lse, sel = m.moba_decode_ref(q[N - 1], k, v, B, topk)
        t = N - 1
        j = t // B
        for h in range(H):
            if j + 1 <= topk:
                want = list(range(j + 1))
            else:
                kbar = _t64(k[:j * B, h]).reshape(j, B, D).mean(dim=1).to(torch.float32).to(torch.float64)
                sc = (kbar @ _t64(q[t, h])).to(torch.float32).to(torch.float64).numpy()
                best, best_sum = None, -math.inf
                for comb in itertools.combinations(range(j), topk - 1):
                    s = sum(sc[i] for i in comb)
                    if s > best_sum:
                        best, best_sum = comb, s
                want = sorted(list(best) + [j])
            assert list(sel[h][sel[h] >= 0]) == want, (N, B, topk, h)
        bo, bl = brute_attention_rows(q, k, v, B, sel, t)
        assert np.allclose(out, bo, atol=1e-12, rtol=0)
        assert np.allclose(lse, bl, atol=1e-12, rtol=0)


def brute_attention_rows(q, k, v, B, sel_t, t):
    """Attention of row t over the keys of its chosen blocks (token by token mask), through SDPA."""
    N, H, D = k.shape
    out = np.zeros((H, D))
    lse = np.zeros(H)
    for h in range(H):
        chosen = set(int(x) for x in sel_t[h] if x >= 0)
        keys = [s for s in range(t + 1) if s // B in chosen]
        out[h], lse[h] = _sdpa_one(q[t, h], k[keys, h], v[keys, h])
    return out, lse


def pin_decode_matches_prefill_row(m):
    """With B dividing N, the decode step is the prefill's last row."""
    for N, H, D, B, topk, seed in [(64, 2, 8, 8, 3, 201), (96, 1, 8, 16, 2, 202), (128, 2, 4, 16, 5, 203)]:
        q, k, v = _rand(N, H, D, seed)
        out, lse, sel = m.moba_decode_ref(q[N - 1], k, v, B, topk)
        po, pl, ps = m.moba_ref(q, k, v, B, topk, rows=np.array([N - 1]))
        assert np.array_equal(sel, ps[:, 0])
        assert np.allclose(out, po[0], atol=1e-13, rtol=0)
        assert np.allclose(lse, pl[:, 0], atol=1e-13, rtol=0)
        kbar = m.pooled_keys_fp32(k, B)
        o2, l2, s2 = m.moba_decode_ref(q[N - 1], k, v, B, topk, kbar32=kbar)
        assert np.array_equal(s2, sel) and np.array_equal(o2, out) and np.array_equal(l2, lse)


# ---------------------------------------------------------------------------
# backward pins
# ---------------------------------------------------------------------------

def _autograd_masked(q, k, v, dout, mask):
    """dq, dk, dv of one head through torch autograd of SDPA (fp64) with a boolean mask."""
    qh, kh, vh = (_t64(x).requires_grad_(True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(qh[None], kh[None], vh[None], attn_mask=mask[None])[0]
    o.backward(_t64(dout))
    return qh.grad.numpy(), kh.grad.numpy(), vh.grad.numpy()


def _brute_mask(sel_h, N, B):
    mask = torch.zeros((N, N), dtype=torch.bool)
    for t in range(N):
        chosen = set(int(x) for x in sel_h[t] if x >= 0)
        for s in range(t + 1):
            if s // B in chosen:
                mask[t, s] = True
    return mask


def pin_backward_full_causal(m):
    """top_k >= n: the gradients of plain causal attention (torch autograd of SDPA)."""
    N, H, D, B = 64, 2, 8, 8
    q, k, v = _rand(N, H, D, 51)
    do = np.random.default_rng(52).standard_normal((N, H, D))
    dq, dk, dv, _ = m.moba_backward_ref(q, k, v, do, B, N // B + 1)
    causal = torch.ones(N, N, dtype=torch.bool).tril()
    for h in range(H):
        rq, rk, rv = _autograd_masked(q[:, h], k[:, h], v[:, h], do[:, h], causal)
        for got, ref in ((dq, rq), (dk, rk), (dv, rv)):
            assert np.allclose(got[:, h], ref, atol=1e-12, rtol=0)


def pin_backward_block_diagonal(m):
    """top_k = 1: the gradients of block-diagonal causal attention."""
    N, H, D, B = 48, 1, 8, 16
    q, k, v = _rand(N, H, D, 53)
    do = np.random.default_rng(54).standard_normal((N, H, D))
    dq, dk, dv, _ = m.moba_backward_ref(q, k, v, do, B, 1)
    blockdiag = torch.tensor([[s // B == t // B and s <= t for s in range(N)] for t in range(N)])
    rq, rk, rv = _autograd_masked(q[:, 0], k[:, 0], v[:, 0], do[:, 0], blockdiag)
    for got, ref in ((dq, rq), (dk, rk), (dv, rv)):
        assert np.allclose(got[:, 0], ref, atol=1e-12, rtol=0)


def pin_backward_brute(m):
    """Tiny inputs: autograd of SDPA under the mask of the exhaustive-search selection, both methods."""
    for N, H, D, B, topk, seed in [(32, 2, 4, 4, 3, 55), (48, 1, 4, 8, 2, 56), (24, 2, 4, 2, 4, 57)]:
        q, k, v = _rand(N, H, D, seed)
        do = np.random.default_rng(seed + 100).standard_normal((N, H, D))
        bsel = brute_selection(q, k, B, topk)
        for method in ("dense", "blocks"):
            dq, dk, dv, _ = m.moba_backward_ref(q, k, v, do, B, topk, method=method)
            for h in range(H):
                rq, rk, rv = _autograd_masked(q[:, h], k[:, h], v[:, h], do[:, h], _brute_mask(bsel[h], N, B))
                for got, ref in ((dq, rq), (dk, rk), (dv, rv)):
                    assert np.allclose(got[:, h], ref, atol=1e-12, rtol=0), (N, B, topk, method)


def pin_backward_finite_difference(m):
    """Directional derivatives of <dO, out> by central differences of the forward oracle
    (selection held fixed), for q, k and v separately."""
    N, H, D, B, topk = 64, 2, 8, 8, 3
    q, k, v = (x.astype(np.float64) for x in _rand(N, H, D, 58))
    rng = np.random.default_rng(59)
    do = rng.standard_normal((N, H, D))
    dq, dk, dv, sel = m.moba_backward_ref(q, k, v, do, B, topk)
    eps = 1e-6
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        u = rng.standard_normal((N, H, D))
        plus = [q, k, v]
        minus = [q, k, v]
        plus[which] = plus[which] + eps * u
        minus[which] = minus[which] - eps * u
        op, _, _ = m.moba_ref(*plus, B, topk, sel=sel)
        om_, _, _ = m.moba_ref(*minus, B, topk, sel=sel)
        fd = np.sum(do * (op - om_)) / (2 * eps)
        an = np.sum(grad * u)
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (which, fd, an)


def pin_backward_invariants(m):
    """Softmax rows sum to one: Σ_keys dK = 0 and Σ_keys dV = Σ_queries dO, per head."""
    N, H, D, B, topk = 128, 3, 8, 16, 3
    q, k, v = _rand(N, H, D, 60)
    do = np.random.default_rng(61).standard_normal((N, H, D))
    for method in ("dense", "blocks"):
        dq, dk, dv, _ = m.moba_backward_ref(q, k, v, do, B, topk, method=method)
        assert np.allclose(dk.sum(axis=0), 0.0, atol=1e-11)
        assert np.allclose(dv.sum(axis=0), do.sum(axis=0), atol=1e-11, rtol=0)


def pin_backward_methods_agree(m):
    """The dense and per-block evaluations agree, also on a subset of heads."""
    N, H, D, B, topk = 256, 3, 16, 32, 3
    q, k, v = _rand(N, H, D, 62)
    do = np.random.default_rng(63).standard_normal((N, H, D))
    a = m.moba_backward_ref(q, k, v, do, B, topk, heads=[2, 0])
    b = m.moba_backward_ref(q, k, v, do, B, topk, heads=[2, 0], method="blocks")
    full = m.moba_backward_ref(q, k, v, do, B, topk)
    for x, y, z in zip(a[:3], b[:3], full[:3]):
        assert np.allclose(x, y, atol=1e-12, rtol=0)
        assert np.allclose(x, z[:, [2, 0]], atol=1e-12, rtol=0)


# ---------------------------------------------------------------------------
# pooling variants and dynamic k
# ---------------------------------------------------------------------------

def _torch_pool(k, B, pooling, weights=None):
    """Block keys through torch (fp64), [n, H, D]: amax, or the weighted average."""
    N, H, D = k.shape
    kt = _t64(k).reshape(N // B, B, H, D)
    if pooling == "max":
        return kt.amax(dim=1)
    wt = _t64(weights).T.reshape(N // B, B, H)                       # [n, B, H]
    return torch.einsum("nbh,nbhd->nhd", wt, kt) / wt.sum(dim=1)[:, :, None]


def pin_pooling_max(m):
    """Max pooling: torch amax per block, and the selection it leads to by exhaustive search."""
    for N, H, D, B, topk, seed in [(32, 2, 4, 4, 3, 71), (48, 1, 4, 8, 2, 72)]:
        q, k, v = _rand(N, H, D, seed)
        ref = _torch_pool(k, B, "max").permute(1, 0, 2).numpy()
        assert np.array_equal(m.pooled_keys(k, B, "max"), ref)
        sel, _ = m.select_blocks(q, k, B, topk, pooling="max")
        kb = _torch_pool(k, B, "max").to(torch.float32).to(torch.float64)
        assert np.array_equal(sel, brute_selection(q, k, B, topk, kbar=kb))
        out, _, _ = m.moba_ref(q, k, v, B, topk, pooling="max")
        bout, _ = brute_attention(q, k, v, B, brute_selection(q, k, B, topk, kbar=kb))
        assert np.allclose(out, bout, atol=1e-12, rtol=0)


def pin_pooling_weighted(m):
    """Weighted pooling: the weighted average through torch; equal weights give the mean,
    one-hot weights pick a key, all-zero weights give zero; the selection by exhaustive search."""
    N, H, D, B, topk = 48, 2, 4, 8, 3
    q, k, v = _rand(N, H, D, 73)
    rng = np.random.default_rng(74)
    w = rng.uniform(0.0, 2.0, (H, N))
    ref = _torch_pool(k, B, "weighted", w).permute(1, 0, 2).numpy()
    assert np.allclose(m.pooled_keys(k, B, "weighted", w), ref, atol=1e-14, rtol=0)
    assert np.array_equal(m.pooled_keys(k, B, "weighted", np.full((H, N), 0.5)), m.pooled_keys(k, B))
    onehot = np.zeros((H, N))
    onehot[:, 3::B] = 1.0
    assert np.array_equal(m.pooled_keys(k, B, "weighted", onehot), np.asarray(k[3::B], np.float64).transpose(1, 0, 2))
    zero = w.copy()
    zero[:, :B] = 0.0
    assert np.all(m.pooled_keys(k, B, "weighted", zero)[:, 0] == 0.0)
    sel, _ = m.select_blocks(q, k, B, topk, pooling="weighted", weights=w)
    kb = _torch_pool(k, B, "weighted", w).to(torch.float32).to(torch.float64)
    assert np.array_equal(sel, brute_selection(q, k, B, topk, kbar=kb))


def pin_topk_for_sparsity(m):
    """Dynamic k reproduces the pages' (context, block_size, top_k) table from its sparsity
    column, and k does not shrink as the context grows."""
    for r in golden()["sparsity_table"]["rows"]:
        assert m.topk_for_sparsity(r["N"], r["block_size"], r["sparsity_percent_1dp"] / 100) == r["top_k"]
    snip = golden()["config_snippet"]
    assert m.topk_for_sparsity(snip["context_length"], snip["block_size"], snip["sparsity_percent_1dp"] / 100) \
        == snip["top_k"]
    ks = [m.topk_for_sparsity(N, 512, 0.953) for N in (512, 4096, 32768, 262144, 1048576)]
    assert ks == sorted(ks) and ks[0] == 1 and ks[-1] == round(0.047 * 2048)


# ---------------------------------------------------------------------------
# packed (varlen) batches
# ---------------------------------------------------------------------------

def pin_varlen_brute(m):
    """Packed batch on tiny inputs: masked SDPA over the whole packed axis with a
    mask that is block-diagonal by sequence, from per-sequence exhaustive
    selections; gradients through autograd of the same masked SDPA."""
    B, topk, H, D = 4, 3, 2, 4
    cu = [0, 16, 16, 40, 48]
    T = cu[-1]
    q, k, v = _rand(T, H, D, 81)
    do = np.random.default_rng(82).standard_normal((T, H, D))
    out, lse, sel = m.moba_ref_varlen(q, k, v, cu, B, topk)
    dq, dk, dv = m.moba_backward_ref_varlen(q, k, v, do, cu, B, topk)
    for h in range(H):
        mask = torch.zeros((T, T), dtype=torch.bool)
        for a, b in zip(cu[:-1], cu[1:]):
            if b == a:
                continue
            bs = brute_selection(q[a:b], k[a:b], B, topk)
            assert np.array_equal(np.where(bs[h] >= 0, bs[h] + a // B, -1), sel[h, a:b])
            mask[a:b, a:b] = _brute_mask(bs[h], b - a, B)
        qh, kh, vh = (_t64(x[:, h]) for x in (q, k, v))
        ref = torch.nn.functional.scaled_dot_product_attention(qh[None], kh[None], vh[None], attn_mask=mask[None])[0]
        assert np.allclose(out[:, h], ref.numpy(), atol=1e-12, rtol=0)
        rl = torch.logsumexp(((qh @ kh.T) / math.sqrt(D)).masked_fill(~mask, -math.inf), -1)
        assert np.allclose(lse[h], rl.numpy(), atol=1e-12, rtol=0)
        rq, rk, rv = _autograd_masked(q[:, h], k[:, h], v[:, h], do[:, h], mask)
        for got, r in ((dq, rq), (dk, rk), (dv, rv)):
            assert np.allclose(got[:, h], r, atol=1e-12, rtol=0)


def pin_varlen_one_sequence_and_order(m):
    """One sequence is the plain prefill; swapping two sequences swaps their outputs."""
    B, topk = 8, 3
    q, k, v = _rand(64, 2, 8, 83)
    o1, l1, s1 = m.moba_ref(q, k, v, B, topk)
    o2, l2, s2 = m.moba_ref_varlen(q, k, v, [0, 64], B, topk)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2) and np.array_equal(s1, s2)
    perm = np.r_[np.arange(40, 64), np.arange(0, 40)]
    oa, la, _ = m.moba_ref_varlen(q, k, v, [0, 40, 64], B, topk)
    ob, lb, _ = m.moba_ref_varlen(q[perm], k[perm], v[perm], [0, 24, 64], B, topk)
    assert np.allclose(oa[perm], ob, atol=1e-12, rtol=0) and np.allclose(la[:, perm], lb, atol=1e-12, rtol=0)


ALL_PINS = [
    pin_bruteforce_tiny, pin_chunked_loops, pin_full_causal, pin_block_diagonal, pin_first_token, pin_constant_v,
    pin_zero_query, pin_invariants, pin_pages_worked_example, pin_pages_sparsity_table,
    pin_granularity, pin_closed_form_pairs, pin_query_lists_hand_example, pin_query_lists_transpose,
    pin_lse_merge, pin_pooling_linearity,
    pin_gate_rounding, pin_row_mode_matches, pin_decode_full_attention, pin_decode_own_block,
    pin_decode_first_token, pin_decode_brute_selection, pin_decode_matches_prefill_row,
    pin_backward_full_causal, pin_backward_block_diagonal, pin_backward_brute, pin_backward_finite_difference,
    pin_backward_invariants, pin_backward_methods_agree, pin_pooling_max, pin_pooling_weighted,
    pin_topk_for_sparsity, pin_varlen_brute, pin_varlen_one_sequence_and_order,
]
