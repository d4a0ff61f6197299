"""Plain fp64 CPU oracle of the MoBA causal prefill forward pass.

TEST INFRASTRUCTURE ONLY. This module is imported by the test-suite, by the
package smoke check and by the benchmark's CPU-baseline leg; the product path
never imports, calls or executes anything here. It shares no code, header,
table or helper with the HIP library.

What it computes (one sequence, H heads, head size D, block size B, n = N/B):

1. Block partition: the context of N tokens is cut into n blocks of B
   contiguous tokens (Moonshot MoBA report as summarised by 智东西,
   section 二 "block partition", B = N/n).
2. Mean-pooled block key K̄_i = mean of the B keys of block i ("score_pooling:
   mean" in the configuration snippet, section 3 of the wzjinhao.cn MoBA
   engineering article; pomoai MoBA overview, "核心原理" step 2).
3. Parameter-less gate: score g_i = <q_t, K̄_i>, no scale, no learned weights
   (same sources; 智东西 section 二, relevance score s_i).
4. Causal top-k: block j = floor(t/B) is always chosen and causally masked;
   among past blocks i < j the k-1 best scores are added; no future block is
   ever chosen (wzjinhao.cn article section 3, the causal_mask and
   current_block_force switches; 智东西 section 二, causality paragraph;
   aliyun article, "MoBA 的技术原理" causality item). The list is returned in
   ascending block order (the block-select snippet of wzjinhao.cn section 4
   sorts its result).
5. Attention over the chosen keys: softmax(q·kᵀ/√D)·v restricted to the
   attended set A(t) (0539edu.com NSA/MoBA explainer, section 1 formula).
   The per-block partial outputs merged by log-sum-exp that the pages describe
   (pomoai overview step 3; 智东西 section 二 steps 3-5) are only a faster route
   to this one softmax, so the oracle evaluates the softmax directly.

Readings of points the pages leave open:

* top_k counts the forced current block (k blocks in total; the configuration
  section of the wzjinhao.cn article says a token sees exactly k blocks and
  derives sparsity 1 - B*k/N from it).
* When fewer than k blocks are eligible (j < k-1) every block 0..j is chosen
  and the selection row is padded with -1.
* Exact score ties are broken toward the lower block index.
* The gate decision is taken in fp32, the precision of the pages' block-select
  snippet (float32 keys and query): K̄ is the exact mean rounded once to fp32,
  and each score is the exact dot product of q with that fp32 K̄, rounded once
  to fp32. Everything else (the attention, the log-sum-exp) is fp64.
* The softmax scale is 1/√D; lse is the natural log of the sum of
  exp(q·k/√D) over A(t).

``moba_backward_ref`` gives the gradients of the prefill output with respect
to q, k and v for a given upstream gradient dO (the pages train and
continually pretrain with MoBA: 智东西 section 三, the scaling-law and hybrid
training experiments). The gate is a top-k choice, piecewise constant in q and
k, so no gradient flows through it or through the block means: the selection
is held fixed and the gradients are those of the masked softmax attention over
A(t) (the textbook softmax Jacobian).

``moba_ref_varlen`` and ``moba_backward_ref_varlen`` take a packed batch of
independent sequences (token offsets ``cu_seqlens``, each length a multiple of
B) and apply the single-sequence definitions to each one.

``query_lists`` regroups a selection into per-block lists of the queries
that chose each past block (the reordering of 智东西 section 二, steps 1-2).

``moba_decode_ref`` is the generation step after the prefill: the newest token
(position N - 1 of a cache whose length need not be a multiple of B, so its
own block may be partial) gated and attended exactly like a prefill row; with
top_k above the number of past blocks it is full attention.
"""

from __future__ import annotations

import math

import numpy as np


def n_blocks(N: int, block_size: int) -> int:
    """Number of blocks n = N / B; the partition needs B to divide N."""
    if block_size < 1 or N < 1 or N % block_size != 0:
        raise ValueError(f"block_size {block_size} must divide N {N}")
    return N // block_size


POOLINGS = ("mean", "max", "weighted")


def pooled_keys(k: np.ndarray, block_size: int, pooling: str = "mean", weights=None) -> np.ndarray:
    """Representative key of every block (fp64): [H, n, D].

    ``k`` is [N, H, D]; its values are widened exactly to fp64. ``pooling``:
    "mean" (the pages' score_pooling), "max" (per-dimension maximum over the
    block's keys) or "weighted" (sum of w_t k_t over the block divided by the
    sum of w_t, with ``weights`` [H, N] non-negative per (head, token); a block
    whose weights are all zero pools to the zero vector). The last two are the
    variants the wzjinhao.cn MoBA article suggests trying in its closing
    section.
    """
    N, H, D = k.shape
    n = n_blocks(N, block_size)
    k64 = np.asarray(k, dtype=np.float64).reshape(n, block_size, H, D)
    if pooling == "mean":
        total = np.zeros((n, H, D), dtype=np.float64)
        for r in range(block_size):          # fixed order, one key of every block at a time
            total += k64[:, r]
        return np.ascontiguousarray((total / block_size).transpose(1, 0, 2))
    if pooling == "max":
        return np.ascontiguousarray(k64.max(axis=1).transpose(1, 0, 2))
    if pooling == "weighted":
        w64 = np.asarray(weights, dtype=np.float64)
        if w64.shape != (H, N) or np.any(w64 < 0):
            raise ValueError("weights must be a non-negative [H, N] array")
        wb = w64.reshape(H, n, block_size).transpose(1, 2, 0)     # [n, B, H]
        total = np.zeros((n, H, D), dtype=np.float64)
        wsum = np.zeros((n, H), dtype=np.float64)
        for r in range(block_size):
            total += wb[:, r, :, None] * k64[:, r]
            wsum += wb[:, r, :]
        safe = np.where(wsum > 0, wsum, 1.0)
        pooled = np.where((wsum > 0)[:, :, None], total / safe[:, :, None], 0.0)
        return np.ascontiguousarray(pooled.transpose(1, 0, 2))
    raise ValueError(f"unknown pooling {pooling!r}")


def pooled_keys_fp32(k: np.ndarray, block_size: int, pooling: str = "mean", weights=None) -> np.ndarray:
    """The block representative keys rounded once to fp32 (the gate's precision): [H, n, D]."""
    return pooled_keys(k, block_size, pooling, weights).astype(np.float32)


def topk_for_sparsity(N: int, block_size: int, sparsity: float) -> int:
    """Dynamic k: the top_k that keeps a late query's sparsity 1 - B k / N at
    ``sparsity`` for this context length, k = round((1 - sparsity) N / B),
    clamped to 1 .. n. The wzjinhao.cn MoBA article lets k grow with the
    context (closing section) and pairs lengths with (block_size, top_k) at
    about constant sparsity in its section 3 table."""
    n = n_blocks(N, block_size)
    if not 0.0 <= sparsity < 1.0:
        raise ValueError("sparsity must be in [0, 1)")
    return int(min(n, max(1, round((1.0 - sparsity) * N / block_size))))


def gate_scores(q_rows: np.ndarray, kbar32_h: np.ndarray) -> np.ndarray:
    """fp32 gate scores of query rows against every block of one head.

    ``q_rows`` [R, D] (one head), ``kbar32_h`` [n, D] fp32 mean keys. The dot
    products are formed in fp64 (exact to fp64 rounding for bf16/fp32 inputs)
    and rounded once to fp32. Returns [R, n] float32; future blocks are not
    masked here.
    """
    s = np.asarray(q_rows, np.float64) @ np.asarray(kbar32_h, np.float64).T
    return s.astype(np.float32)


def select_row(scores_row: np.ndarray, j: int, topk: int) -> list[int]:
    """Causal top-k for one query in block j from its fp32 block scores.

    Returns the chosen blocks in ascending order: block j plus the k-1 highest
    scoring past blocks, ranked by score (descending) then block index
    (ascending); all of 0..j when j+1 <= k.
    """
    if j + 1 <= topk:
        return list(range(j + 1))
    past = [(-float(scores_row[i]), i) for i in range(j)]
    past.sort()
    chosen = [i for _, i in past[:topk - 1]]
    return sorted(chosen + [j])


def select_blocks(q: np.ndarray, k: np.ndarray, block_size: int, topk: int,
                  rows: np.ndarray | None = None, chunk: int = 65536, pooling: str = "mean", weights=None):
    """Selection of every (head, row): int32 [H, R, topk], ascending, -1 padded.

    ``rows`` defaults to all N query rows; ``pooling``/``weights`` pick the
    block representative key (see ``pooled_keys``). Also returns the fp32
    pooled keys.
    """
    N, H, D = q.shape
    n = n_blocks(N, block_size)
    if topk < 1:
        raise ValueError("topk must be >= 1")
    kbar32 = pooled_keys_fp32(k, block_size, pooling, weights)
    rows = np.arange(N, dtype=np.int64) if rows is None else np.asarray(rows, np.int64)
    R = rows.shape[0]
    sel = np.full((H, R, topk), -1, dtype=np.int32)
    for h in range(H):
        for c0 in range(0, R, chunk):
            rr = rows[c0:c0 + chunk]
            sc = gate_scores(q[rr, h, :], kbar32[h])          # [r, n]
            jj = rr // block_size
            neg = -sc.astype(np.float64)
            neg[np.arange(n)[None, :] >= jj[:, None]] = np.inf   # only past blocks compete
            order = np.argsort(neg, axis=1, kind="stable")       # ties keep lower index first
            for i, (t, j) in enumerate(zip(rr, jj)):
                if j + 1 <= topk:
                    row = list(range(j + 1))
                else:
                    row = sorted(order[i, :topk - 1].tolist() + [int(j)])
                sel[h, c0 + i, :len(row)] = row
    return sel, kbar32


def query_lists(sel: np.ndarray, block_size: int):
    """Queries regrouped by the past block they chose.

    Attention runs block by block over the queries routed to each block once
    the queries are reordered by their block assignment (智东西 report,
    section 二, implementation steps 1-2). For every head h and block b, in
    (h, b) order, the list holds the query positions t, ascending, whose
    selection row sel[h, t] contains b as a past block (b < t // block_size);
    a query's own block is left out, its queries being that block's tokens.

    Returns (offs, qidx): list (h, b) is qidx[offs[h*n + b]:offs[h*n + b + 1]],
    offs int64 [H*n + 1], qidx int32.
    """
    H, N, _ = sel.shape
    n = n_blocks(N, block_size)
    lists = [[[] for _ in range(n)] for _ in range(H)]
    for h in range(H):
        for t in range(N):                      # ascending t: every list comes out ascending
            j = t // block_size
            for b in sel[h, t]:
                b = int(b)
                if 0 <= b < j:
                    lists[h][b].append(t)
    offs = [0]
    qidx: list[int] = []
    for h in range(H):
        for b in range(n):
            qidx.extend(lists[h][b])
            offs.append(len(qidx))
    return np.asarray(offs, np.int64), np.asarray(qidx, np.int32)


def attended_keys(sel_row, t: int, block_size: int) -> np.ndarray:
    """Key positions A(t): every chosen past block in full, the own block up to t."""
    j = t // block_size
    parts = []
    for b in sel_row:
        b = int(b)
        if b < 0:
            continue
        if b < j:
            parts.append(np.arange(b * block_size, (b + 1) * block_size))
        elif b == j:
            parts.append(np.arange(j * block_size, t + 1))
        else:
            raise ValueError(f"future block {b} chosen for row {t}")
    return np.concatenate(parts)


def _softmax_rows(logits: np.ndarray):
    m = np.max(logits, axis=-1, keepdims=True)
    p = np.exp(logits - m)
    l = np.sum(p, axis=-1, keepdims=True)
    return p / l, (m + np.log(l))[..., 0]


def _attend_dense(q, k, v, block_size, sel, rows, out, lse, scale, max_rows_chunk):
    """Dense masked form: per query block j, logits against every key of blocks
    0..j, masked to A(t), softmax, then the product with V."""
    N, H, D = q.shape
    n = N // block_size
    B = block_size
    for h in range(H):
        for j in range(n):
            in_j = np.nonzero(rows // B == j)[0]          # indices into rows
            if in_j.size == 0:
                continue
            nk = (j + 1) * B
            kh = np.asarray(k[:nk, h, :], np.float64)
            vh = np.asarray(v[:nk, h, :], np.float64)
            key_block = np.arange(nk) // B
            key_pos = np.arange(nk)
            for c0 in range(0, in_j.size, max_rows_chunk):
                idx = in_j[c0:c0 + max_rows_chunk]
                t = rows[idx]
                chosen = np.zeros((idx.size, n), dtype=bool)
                for i, r in enumerate(idx):
                    srow = sel[h, r]
                    chosen[i, srow[srow >= 0]] = True
                mask = chosen[:, key_block] & (key_pos[None, :] <= t[:, None])
                logits = (np.asarray(q[t, h, :], np.float64) @ kh.T) * scale
                logits = np.where(mask, logits, -np.inf)
                p, l = _softmax_rows(logits)
                out[idx, h] = p @ vh
                lse[h, idx] = l


def _attend_by_block(q, k, v, block_size, sel, rows, out, lse, scale):
    """Softmax over A(t) for selected rows, with the logits of each chosen
    block formed by one matrix product over the rows that chose it: a first
    pass takes the row maxima over A(t), a second the exponentials, their sum
    and the weighted sum of V."""
    N, H, D = q.shape
    B = block_size
    R = rows.shape[0]
    jrow = rows // B
    for h in range(H):
        qh = np.asarray(q[rows, h, :], np.float64)
        s = sel[h]                                        # [R, topk]
        blocks = np.unique(s[s >= 0])
        groups = []
        for b in blocks:
            ridx = np.nonzero((s == b).any(axis=1))[0]
            own = jrow[ridx] == b                          # the row's own block: keys up to t
            groups.append((int(b), ridx, own))

        def logits_of(b, ridx, own, kb):
            lg = (qh[ridx] @ kb.T) * scale
            if own.any():
                kpos = b * B + np.arange(B)
                lg[own] = np.where(kpos[None, :] <= rows[ridx][own][:, None], lg[own], -np.inf)
            return lg

        m = np.full(R, -np.inf)
        for b, ridx, own in groups:
            kb = np.asarray(k[b * B:(b + 1) * B, h, :], np.float64)
            m[ridx] = np.maximum(m[ridx], logits_of(b, ridx, own, kb).max(axis=1))
        l = np.zeros(R)
        acc = np.zeros((R, D))
        for b, ridx, own in groups:
            kb = np.asarray(k[b * B:(b + 1) * B, h, :], np.float64)
            vb = np.asarray(v[b * B:(b + 1) * B, h, :], np.float64)
            p = np.exp(logits_of(b, ridx, own, kb) - m[ridx][:, None])
            l[ridx] += p.sum(axis=1)
            acc[ridx] += p @ vb
        out[:, h] = acc / l[:, None]
        lse[h] = m + np.log(l)


def _attend_rowwise(q, k, v, block_size, sel, rows, out, lse, scale):
    """One query at a time over its gathered key set A(t)."""
    N, H, D = q.shape
    for h in range(H):
        for i, t in enumerate(rows):
            keys = attended_keys(sel[h, i], int(t), block_size)
            kh = np.asarray(k[keys, h, :], np.float64)
            vh = np.asarray(v[keys, h, :], np.float64)
            logits = (kh @ np.asarray(q[t, h], np.float64)) * scale
            p, l = _softmax_rows(logits[None, :])
            out[i, h] = p[0] @ vh
            lse[h, i] = l[0]


def moba_ref(q, k, v, block_size: int, topk: int, sel=None, rows=None, method: str | None = None,
             max_rows_chunk: int = 512, pooling: str = "mean", weights=None):
    """fp64 MoBA causal prefill.

    Arguments are [N, H, D] arrays (float32 holding exact bf16 or fp32 values).
    ``sel`` optionally overrides the gate ([H, R, topk] int32 for the same rows).
    ``rows`` selects the query rows to evaluate (default: all).
    ``pooling``/``weights`` pick the gate's block key (see ``pooled_keys``).
    ``method`` picks one of three evaluations of the same softmax over A(t):
    "dense" (masked logits against all keys up to the row's block; the default
    for all rows), "blocks" (logits of each chosen block for the rows that
    chose it; the default for sampled rows) or "rowwise" (gathered keys, one
    row at a time).

    Returns ``(out, lse, sel)``: out [R, H, D] fp64, lse [H, R] fp64 (natural
    log), sel [H, R, topk] int32.
    """
    q = np.asarray(q)
    N, H, D = q.shape
    n_blocks(N, block_size)
    all_rows = rows is None
    rows = np.arange(N, dtype=np.int64) if all_rows else np.asarray(rows, np.int64)
    if sel is None:
        sel, _ = select_blocks(q, k, block_size, topk, rows=None if all_rows else rows, pooling=pooling,
                               weights=weights)
    if method is None:
        method = "dense" if all_rows else "blocks"
    scale = 1.0 / math.sqrt(D)
    R = rows.shape[0]
    out = np.zeros((R, H, D), np.float64)
    lse = np.zeros((H, R), np.float64)
    if method == "dense":
        _attend_dense(q, k, v, block_size, sel, rows, out, lse, scale, max_rows_chunk)
    elif method == "blocks":
        _attend_by_block(q, k, v, block_size, sel, rows, out, lse, scale)
    elif method == "rowwise":
        _attend_rowwise(q, k, v, block_size, sel, rows, out, lse, scale)
    else:
        raise ValueError(method)
    return out, lse, sel


def attended_count(t: int, block_size: int, topk: int) -> int:
    """|A(t)| for a row whose selection has min(k, j+1) blocks: c(t)."""
    j = t // block_size
    return min(topk - 1, j) * block_size + (t % block_size) + 1


def attended_pairs_closed_form(N: int, block_size: int, topk: int) -> int:
    """Σ_t |A(t)| for one head, in closed form.

    Rows in blocks j < k-1 see all j past blocks, later rows see k-1 of them;
    each row also sees its own block up to itself.
    """
    n = n_blocks(N, block_size)
    B, k = block_size, topk
    m = min(k - 1, n)                     # blocks j = 0..m-1 see j past blocks
    past = B * B * (m * (m - 1) // 2) + B * B * max(n - m, 0) * (k - 1)
    own = n * B * (B + 1) // 2
    return past + own


def sparsity(N: int, block_size: int, topk: int) -> float:
    """Fraction of the context a late query does not attend: 1 - B*k/N."""
    return 1.0 - block_size * min(topk, n_blocks(N, block_size)) / N


def moba_decode_ref(q_new, k, v, block_size: int, topk: int, kbar32=None, sel=None):
    """fp64 MoBA decode step: the newest token attends its selected blocks.

    The generation step after the prefill (wzjinhao.cn MoBA article, section 3:
    decoding may switch back to full attention; the MoBA form gates the new
    token exactly like a prefill row). ``q_new`` is [H, D], the query of the
    token at position t = N - 1, whose key and value are already the last rows
    of the cache ``k``, ``v`` [N, H, D]; N need not be a multiple of B, so the
    token's own block j = floor(t / B) may be partial (keys jB .. t).

    Gate: the fp32 mean keys of the complete past blocks 0 .. j-1 (``kbar32``
    [H, >= j, D] if given, else the exact mean rounded once to fp32), fp32
    scores, then the same causal top-k as a prefill row (``select_row``).
    top_k > j selects every past block: full causal attention for the token.

    Returns ``(out [H, D] fp64, lse [H] fp64 natural log, sel [H, topk] int32)``.
    """
    k = np.asarray(k)
    N, H, D = k.shape
    if N < 1 or block_size < 1 or topk < 1:
        raise ValueError("need N >= 1, block_size >= 1, topk >= 1")
    t = N - 1
    j = t // block_size
    if sel is None:
        if kbar32 is None and j > 0:
            kbar32 = pooled_keys_fp32(k[:j * block_size], block_size)
        sel = np.full((H, topk), -1, dtype=np.int32)
        for h in range(H):
            scores = gate_scores(np.asarray(q_new)[h][None, :], kbar32[h, :j])[0] if j > 0 else np.zeros(0, np.float32)
            row = select_row(scores, j, topk)
            sel[h, :len(row)] = row
    inv_sqrt_d = 1.0 / math.sqrt(D)
    out = np.zeros((H, D), np.float64)
    lse = np.zeros(H, np.float64)
    for h in range(H):
        keys = attended_keys(sel[h], t, block_size)
        k_att = np.asarray(k[keys, h, :], np.float64)
        v_att = np.asarray(v[keys, h, :], np.float64)
        logits = (k_att @ np.asarray(q_new[h], np.float64)) * inv_sqrt_d
        p, l = _softmax_rows(logits[None, :])
        out[h] = p[0] @ v_att
        lse[h] = l[0]
    return out, lse, sel


def _backward_dense(q, k, v, dout, block_size, sel, heads, dq, dk, dv, scale):
    """Dense masked form, per (head, query block j): the logits of the block's
    rows against every key of blocks 0..j, masked to A(t), softmax P, then
    dV += Pᵀ dO, dP = dO Vᵀ, dL = P (dP - Σ_keys P dP), dQ = scale dL K,
    dK += scale dLᵀ Q."""
    N, H, D = q.shape
    n = N // block_size
    B = block_size
    for oh, h in enumerate(heads):
        for j in range(n):
            t = np.arange(j * B, (j + 1) * B)
            nk = (j + 1) * B
            qh = np.asarray(q[t, h, :], np.float64)
            doh = np.asarray(dout[t, h, :], np.float64)
            kh = np.asarray(k[:nk, h, :], np.float64)
            vh = np.asarray(v[:nk, h, :], np.float64)
            chosen = np.zeros((B, n), dtype=bool)
            for i, r in enumerate(t):
                srow = sel[h, r]
                chosen[i, srow[srow >= 0]] = True
            key_pos = np.arange(nk)
            mask = chosen[:, key_pos // B] & (key_pos[None, :] <= t[:, None])
            logits = np.where(mask, (qh @ kh.T) * scale, -np.inf)
            p, _ = _softmax_rows(logits)
            dp = doh @ vh.T
            dl = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
            dq[t, oh] = scale * (dl @ kh)
            dk[:nk, oh] += scale * (dl.T @ qh)
            dv[:nk, oh] += p.T @ doh


def _backward_by_block(q, k, v, dout, block_size, sel, heads, dq, dk, dv, scale):
    """The same gradients with the logits of each chosen block formed only for
    the rows that chose it: a first pass gives every row's softmax maximum and
    denominator over A(t), a second the row sums Σ_keys P dP, a third the
    gradient terms of each block."""
    N, H, D = q.shape
    B = block_size
    rows = np.arange(N)
    jrow = rows // B
    for oh, h in enumerate(heads):
        qh = np.asarray(q[:, h, :], np.float64)
        doh = np.asarray(dout[:, h, :], np.float64)
        s = sel[h]
        groups = []
        for b in np.unique(s[s >= 0]):
            ridx = np.nonzero((s == b).any(axis=1))[0]
            groups.append((int(b), ridx, jrow[ridx] == b))

        def probs_of(b, ridx, own, m, l):
            kb = np.asarray(k[b * B:(b + 1) * B, h, :], np.float64)
            lg = (qh[ridx] @ kb.T) * scale
            if own.any():
                kpos = b * B + np.arange(B)
                lg[own] = np.where(kpos[None, :] <= ridx[own][:, None], lg[own], -np.inf)
            if m is None:
                return lg
            return np.exp(lg - m[ridx][:, None]) / l[ridx][:, None]

        m = np.full(N, -np.inf)
        for b, ridx, own in groups:
            m[ridx] = np.maximum(m[ridx], probs_of(b, ridx, own, None, None).max(axis=1))
        l = np.zeros(N)
        for b, ridx, own in groups:
            l[ridx] += np.exp(probs_of(b, ridx, own, None, None) - m[ridx][:, None]).sum(axis=1)
        delta = np.zeros(N)
        for b, ridx, own in groups:
            vb = np.asarray(v[b * B:(b + 1) * B, h, :], np.float64)
            p = probs_of(b, ridx, own, m, l)
            delta[ridx] += np.sum(p * (doh[ridx] @ vb.T), axis=1)
        for b, ridx, own in groups:
            kb = np.asarray(k[b * B:(b + 1) * B, h, :], np.float64)
            vb = np.asarray(v[b * B:(b + 1) * B, h, :], np.float64)
            p = probs_of(b, ridx, own, m, l)
            dl = p * (doh[ridx] @ vb.T - delta[ridx][:, None])
            dq[ridx, oh] += scale * (dl @ kb)
            dk[b * B:(b + 1) * B, oh] += scale * (dl.T @ qh[ridx])
            dv[b * B:(b + 1) * B, oh] += p.T @ doh[ridx]


def moba_backward_ref(q, k, v, dout, block_size: int, topk: int, sel=None, heads=None, method: str = "dense",
                      pooling: str = "mean", weights=None):
    """fp64 gradients of the MoBA causal prefill output.

    ``dout`` [N, H, D] is the upstream gradient of ``out``; the lse output
    carries none. The selection (``sel`` [H, N, topk], default: the oracle's
    own gate) is held fixed: the top-k choice has no gradient. ``heads``
    limits the work to some heads (default: all). ``method`` is "dense" (the
    masked form per query block) or "blocks" (the logits of each chosen block
    for the rows that chose it).

    Returns ``(dq, dk, dv, sel)``: gradients [N, len(heads), D] fp64.
    """
    q = np.asarray(q)
    N, H, D = q.shape
    n_blocks(N, block_size)
    if sel is None:
        sel, _ = select_blocks(q, k, block_size, topk, pooling=pooling, weights=weights)
    heads = list(range(H)) if heads is None else [int(h) for h in heads]
    softmax_scale = 1.0 / math.sqrt(D)
    dq = np.zeros((N, len(heads), D), np.float64)
    dk = np.zeros((N, len(heads), D), np.float64)
    dv = np.zeros((N, len(heads), D), np.float64)
    if method == "dense":
        _backward_dense(q, k, v, dout, block_size, sel, heads, dq, dk, dv, softmax_scale)
    elif method == "blocks":
        _backward_by_block(q, k, v, dout, block_size, sel, heads, dq, dk, dv, softmax_scale)
    else:
        raise ValueError(method)
    return dq, dk, dv, sel


def _segments(cu_seqlens, block_size: int):
    cu = [int(x) for x in cu_seqlens]
    if len(cu) < 2 or cu[0] != 0:
        raise ValueError("cu_seqlens must start at 0 and hold num_seqs + 1 offsets")
    segs = []
    for a, b in zip(cu[:-1], cu[1:]):
        if b < a or (b - a) % block_size != 0:
            raise ValueError("sequence lengths must be non-negative multiples of block_size")
        segs.append((a, b))
    return segs


def moba_ref_varlen(q, k, v, cu_seqlens, block_size: int, topk: int):
    """Packed (varlen) batch: independent sequences concatenated along the token
    axis, cu_seqlens their token offsets. Each sequence is its own MoBA prefill
    (its blocks start at its first token; its queries see only its blocks):
    out [T, H, D], lse [H, T] and sel [H, T, topk] with global block indices."""
    q = np.asarray(q)
    T, H, D = q.shape
    out = np.zeros((T, H, D), np.float64)
    lse = np.zeros((H, T), np.float64)
    sel = np.full((H, T, topk), -1, np.int32)
    for a, b in _segments(cu_seqlens, block_size):
        if b == a:
            continue
        o, l, s = moba_ref(q[a:b], k[a:b], v[a:b], block_size, topk)
        out[a:b] = o
        lse[:, a:b] = l
        sel[:, a:b] = np.where(s >= 0, s + a // block_size, -1)
    return out, lse, sel


def moba_backward_ref_varlen(q, k, v, dout, cu_seqlens, block_size: int, topk: int, sel=None):
    """Gradients of ``moba_ref_varlen``: every sequence on its own. ``sel``
    (global block indices, [H, T, topk]) optionally fixes the selection."""
    q = np.asarray(q)
    T, H, D = q.shape
    grads = [np.zeros((T, H, D), np.float64) for _ in range(3)]
    for a, b in _segments(cu_seqlens, block_size):
        if b == a:
            continue
        s = None if sel is None else np.where(sel[:, a:b] >= 0, sel[:, a:b] - a // block_size, -1)
        dq, dk, dv, _ = moba_backward_ref(q[a:b], k[a:b], v[a:b], dout[a:b], block_size, topk, sel=s)
        for g, x in zip(grads, (dq, dk, dv)):
            g[a:b] = x
    return tuple(grads)
