"""GPU parity: the HIP path through the C-ABI against the fp64 oracle.

Selections must match the oracle bit for bit except on near-ties (see
tests/parity.py); outputs must stay within max-abs tolerances: 2e-2 (bf16 in,
fp32 accumulate) and 1e-4 (fp32 in); lse within 1e-2 / 1e-5.
"""

import numpy as np
import pytest

from block_sparse_long_gating_amd import synth
from tests.parity import LSE_TOL, OUT_TOL, compare_selection, log, max_abs, to_device

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moba():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import block_sparse_long_gating_amd as m
    m.load_library()
    return m


# (N, H, D, B, topk, dtype, seed): several gate tiles and work items, ragged
# query lists, B = 64 (a gate tile spans two blocks), N % 128 != 0, n = 1,
# topk = 1, topk >= n (full causal attention), D = 64.
SMALL = [
    (2048, 2, 128, 256, 3, "bf16", 1),
    (1536, 3, 128, 128, 4, "bf16", 2),
    (4096, 1, 64, 512, 2, "bf16", 3),
    (640, 2, 128, 64, 5, "bf16", 4),
    (320, 1, 128, 64, 3, "bf16", 5),
    (256, 2, 128, 256, 3, "bf16", 6),
    (1024, 2, 128, 128, 1, "bf16", 7),
    (1024, 1, 128, 128, 8, "bf16", 8),
    (1024, 1, 128, 128, 20, "bf16", 9),
    (2048, 1, 128, 64, 12, "bf16", 10),
    (2048, 1, 64, 256, 3, "fp32", 11),
    (1024, 2, 128, 128, 4, "fp32", 12),
    (640, 1, 64, 64, 5, "fp32", 13),
    (4096, 1, 128, 64, 32, "bf16", 14),
    (1024, 40, 64, 128, 4, "bf16", 15),      # many heads, not a power of two
    (1920, 2, 128, 320, 3, "bf16", 16),      # own tiles of 256 + 64 queries, 5 key tiles per block
    (1536, 2, 128, 192, 4, "bf16", 17),      # own tiles of 192 queries, 3 key tiles per block
    (2048, 1, 64, 64, 40, "fp32", 18),       # topk > n = 32: full causal attention, separate merge, fp32
    (1024, 2, 128, 64, 300, "bf16", 19),     # topk far above n = 16: the dense path
]


def _ids(c):
    return "N{}_H{}_D{}_B{}_k{}_{}".format(*c[:6])


def run_case(moba, q, k, v, B, topk, dtype, rows=None, full_out=True):
    from oracle import moba_ref, pooled_keys_fp32, select_blocks
    N, H, D = q.shape
    qd, kd, vd = (to_device(x, dtype) for x in (q, k, v))
    log(f"  gpu: block_mean_keys N={N} H={H} D={D} B={B}")
    kbar = moba.block_mean_keys(kd, B)
    log(f"  gpu: gate_topk topk={topk}")
    sel = moba.gate_topk(qd, kd, B, topk)
    log(f"  gpu: prefill")
    out, lse = moba.prefill(qd, kd, vd, B, topk)
    torch.cuda.synchronize()
    log("  gpu: done")

    ref_kbar = pooled_keys_fp32(k, B)
    kb = kbar.cpu().numpy()
    assert np.max(np.abs(kb - ref_kbar) / np.maximum(np.abs(ref_kbar), 1e-30)) <= 1e-6
    kbar_exact = float(np.mean(kb == ref_kbar))

    gsel = sel.cpu().numpy()
    ref_sel, _ = select_blocks(q, k, B, topk)
    cmp = compare_selection(gsel, ref_sel, q, k, B, topk)
    assert not cmp["bad"], f"selection mismatches beyond near-ties: {cmp['bad'][:5]}"

    if rows is None:
        rows = np.arange(N)
    rows = np.asarray(rows)
    method = "dense" if (full_out and N * H <= 8192) else "blocks"
    ref_out, ref_lse, _ = moba_ref(q, k, v, B, topk, sel=gsel[:, rows], rows=rows, method=method)
    got_out = out.float().cpu().numpy()[rows]
    got_lse = lse.cpu().numpy()[:, rows]
    e_out, e_lse = max_abs(got_out, ref_out), max_abs(got_lse, ref_lse)
    log(f"  sel mismatch rows {cmp['mismatch']} (exempt {cmp['exempt']}, row-max rule {cmp['exempt_rowmax']}), kbar bit-exact {kbar_exact:.4f}, "
        f"max|out| err {e_out:.3e}, max|lse| err {e_lse:.3e}")
    assert e_out <= OUT_TOL[dtype], e_out
    assert e_lse <= LSE_TOL[dtype], e_lse
    assert np.all(np.isfinite(got_out))
    return out, lse, sel


@pytest.mark.parametrize("case", SMALL, ids=_ids)
def test_prefill_small(moba, case):
    N, H, D, B, topk, dtype, seed = case
    log(f"case {_ids(case)}")
    q, k, v = synth.make_qkv(N, H, D, seed=[100, seed], dtype=dtype)
    run_case(moba, q, k, v, B, topk, dtype)


def test_structured_inputs(moba):
    """Zero queries (every gate score ties: the lower-index rule decides) and
    constant values (the output is that constant)."""
    N, H, D, B, topk = 1024, 2, 128, 128, 3
    q, k, v = synth.make_qkv(N, H, D, seed=[101, 0], dtype="bf16")
    q0 = np.zeros_like(q)
    log("case zero-q")
    _, _, sel = run_case(moba, q0, k, v, B, topk, "bf16")
    s = sel.cpu().numpy()
    for t in range(B * 3, N, 97):
        j = t // B
        assert list(s[0, t]) == [0, 1, j]
    vc = np.broadcast_to(synth.round_to_bf16(np.linspace(-2, 2, D, dtype=np.float32)), (N, H, D)).copy()
    log("case constant-v")
    out, _, _ = run_case(moba, q, k, vc, B, topk, "bf16")
    assert max_abs(out.float().cpu().numpy(), vc) <= 2e-2


WORKLOAD_ROWS = {"tiny": None, "c32k": None, "h32": 4096, "n128k": 4096, "m1": 4096}


@pytest.mark.parametrize("name", list(WORKLOAD_ROWS))
def test_workload(moba, name):
    log(f"workload {name}")
    w, q, k, v = synth.make_workload(name)
    count = WORKLOAD_ROWS[name]
    rows = None if count is None else synth.sample_rows(w.N, count, synth.SAMPLE_SEED[name])
    run_case(moba, q, k, v, w.block_size, w.topk, w.dtype, rows=rows, full_out=(count is None))


# (N, H, D, B, topk, seed): several gate tiles, a ragged last tile
# (N % 128 = 64) with B = 64 (a tile spans two blocks), topk = 1 (every list
# empty), topk > n (every past block listed) and the largest ranked topk.
LISTS = [
    (2048, 2, 128, 256, 3, 31),
    (2368, 3, 64, 64, 5, 32),
    (1024, 2, 128, 128, 1, 33),
    (1024, 1, 64, 64, 40, 34),
    (8192, 1, 128, 128, 32, 35),
]


def _lists_from_selection(sel, B):
    """The lists a selection defines, by a stable sort of (head, block, query)
    keys over its (query, past block) pairs (test code, independent of the
    oracle's loops)."""
    H, N, _ = sel.shape
    n = N // B
    t = np.broadcast_to(np.arange(N, dtype=np.int64)[None, :, None], sel.shape)
    h = np.broadcast_to(np.arange(H, dtype=np.int64)[:, None, None], sel.shape)
    keep = (sel >= 0) & (sel < t // B)
    e = h[keep] * n + sel[keep]
    tk = t[keep]
    order = np.lexsort((tk, e))
    offs = np.concatenate([[0], np.cumsum(np.bincount(e, minlength=H * n))])
    return offs, tk[order]


def _check_lists(moba, qd, kd, B, topk):
    """Runs moba_block_query_lists; checks its selection against the gate entry
    point and its lists against the selection (every pair once, ascending,
    closed-form total). Returns the selection and lists on the host."""
    H, N = qd.shape[1], qd.shape[0]
    log(f"  gpu: block_query_lists N={N} H={H} B={B} topk={topk}")
    sel, offs, qidx = moba.block_query_lists(qd, kd, B, topk)
    sel_gate = moba.gate_topk(qd, kd, B, topk)
    torch.cuda.synchronize()
    gsel, goffs, gq = sel.cpu().numpy(), offs.cpu().numpy().astype(np.int64), qidx.cpu().numpy()
    assert np.array_equal(gsel, sel_gate.cpu().numpy())
    n = N // B
    assert goffs[-1] == H * sum(B * min(topk - 1, j) for j in range(n)) == gq.shape[0]
    toffs, tq = _lists_from_selection(gsel, B)
    assert np.array_equal(goffs, toffs)
    assert np.array_equal(gq, tq)
    return gsel, goffs, gq


@pytest.mark.parametrize("case", LISTS, ids=lambda c: "N{}_H{}_D{}_B{}_k{}".format(*c[:5]))
def test_query_lists(moba, case):
    """The regrouped query lists (the queries of every past block, ascending)
    against the oracle's regrouping of the oracle's selection; rows where the
    two selections differ (near-ties only) are left out of both."""
    from oracle import query_lists, select_blocks
    N, H, D, B, topk, seed = case
    log(f"case lists {case}")
    q, k, _ = synth.make_qkv(N, H, D, seed=[seed, 0], dtype="bf16")
    qd, kd = to_device(q, "bf16"), to_device(k, "bf16")
    gsel, goffs, gq = _check_lists(moba, qd, kd, B, topk)
    ref_sel, _ = select_blocks(q, k, B, topk)
    cmp = compare_selection(gsel, ref_sel, q, k, B, topk)
    assert not cmp["bad"], cmp["bad"][:5]
    ref_offs, ref_q = query_lists(ref_sel, B)
    differ = np.any(gsel != ref_sel, axis=2)            # [H, N]
    n = N // B
    for e in range(H * n):
        got = gq[goffs[e]:goffs[e + 1]]
        want = ref_q[ref_offs[e]:ref_offs[e + 1]]
        hd = differ[e // n]
        assert np.array_equal(got[~hd[got]], want[~hd[want]]), e
    log(f"  lists: {goffs[-1]} pairs, {int(differ.sum())} near-tie rows left out")


def test_query_lists_h32(moba):
    """Query lists of the h32 workload (32 heads, 32768 tokens, 64 blocks of
    512, top-3): the transpose of the selection, with the selection checked
    against the oracle on sampled rows."""
    from oracle import select_blocks
    w, q, k, _ = synth.make_workload("h32")
    qd, kd = to_device(q, "bf16"), to_device(k, "bf16")
    gsel, goffs, _ = _check_lists(moba, qd, kd, w.block_size, w.topk)
    rows = synth.sample_rows(w.N, 2048, synth.SAMPLE_SEED["h32"])
    ref_sel, _ = select_blocks(q, k, w.block_size, w.topk, rows=rows)
    cmp = compare_selection(gsel[:, rows], ref_sel, q, k, w.block_size, w.topk, rows=rows)
    assert not cmp["bad"], cmp["bad"][:5]
    log(f"  h32 lists: {goffs[-1]} pairs, sampled sel mismatch {cmp['mismatch']} (exempt {cmp['exempt']})")


def test_needles_are_found(moba):
    """The planted needle blocks of the 128K workload are chosen far more often
    than an average past block."""
    w, q, k, v, ex = synth.make_workload("n128k", with_extras=True)
    sel = moba.gate_topk(to_device(q, "bf16"), to_device(k, "bf16"), w.block_size, w.topk).cpu().numpy()
    base = (w.topk - 1) / (w.n_blocks - 1)
    for h, needles in enumerate(ex["needle_blocks"]):
        late = sel[h, (w.n_blocks - 1) * w.block_size:]
        hits = float(np.isin(late, needles).sum()) / (late.shape[0] * len(needles))
        log(f"  head {h}: needle hit rate {hits:.3f} vs average past block {base:.3f}")
        assert hits > base, (h, hits, base)


def test_deterministic(moba):
    N, H, D, B, topk = 4096, 4, 128, 256, 4
    q, k, v = synth.make_qkv(N, H, D, seed=[102, 0], dtype="bf16")
    qd, kd, vd = (to_device(x, "bf16") for x in (q, k, v))
    o1, l1 = moba.prefill(qd, kd, vd, B, topk)
    o2, l2 = moba.prefill(qd, kd, vd, B, topk)
    s1 = moba.gate_topk(qd, kd, B, topk)
    s2 = moba.gate_topk(qd, kd, B, topk)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))
    assert torch.equal(s1, s2)


def test_stage_events(moba):
    """The timed entry point: same results with all, some or no stage events."""
    N, H, D, B, topk = 4096, 2, 128, 256, 3
    q, k, v = synth.make_qkv(N, H, D, seed=[104, 0], dtype="bf16")
    qd, kd, vd = (to_device(x, "bf16") for x in (q, k, v))
    o1, l1 = moba.prefill(qd, kd, vd, B, topk)
    full = moba.StageEvents()
    o2, l2 = moba.prefill(qd, kd, vd, B, topk, events=full)
    part = moba.StageEvents(stages=("attn_past",))
    o3, l3 = moba.prefill(qd, kd, vd, B, topk, events=part)
    torch.cuda.synchronize()
    full.accumulate()
    part.accumulate()
    for o, l in ((o2, l2), (o3, l3)):
        assert torch.equal(o1.view(torch.int16), o.view(torch.int16))
        assert torch.equal(l1.view(torch.int32), l.view(torch.int32))
    assert all(full.totals[s] >= 0.0 for s in moba.STAGES) and full.totals["attn_past"] > 0.0
    assert part.totals["attn_past"] > 0.0 and part.totals["gate"] == 0.0
    full.close()
    part.close()


def test_bad_arguments_leave_outputs_untouched(moba):
    N, H, D = 1024, 1, 128
    q = torch.zeros(N, H, D, dtype=torch.bfloat16, device="cuda")
    out = torch.full_like(q, 7.0)
    lse = torch.full((H, N), 5.0, device="cuda")
    with pytest.raises(moba.MobaError) as e:
        moba.prefill(q, q, q, 100, 3, out=out, lse=lse)     # block size does not divide N
    assert e.value.status == 1
    q2 = torch.zeros(960, H, D, dtype=torch.bfloat16, device="cuda")
    out2 = torch.full_like(q2, 7.0)
    lse2 = torch.full((H, 960), 5.0, device="cuda")
    with pytest.raises(moba.MobaError) as e:
        moba.prefill(q2, q2, q2, 96, 3, out=out2, lse=lse2)  # block size not a multiple of 64
    assert e.value.status == 2
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()) and bool((lse == 5.0).all())
    assert bool((out2 == 7.0).all()) and bool((lse2 == 5.0).all())


def test_streams(moba):
    """Work is enqueued on the caller's current stream."""
    N, H, D, B, topk = 2048, 2, 128, 256, 3
    q, k, v = synth.make_qkv(N, H, D, seed=[103, 0], dtype="bf16")
    qd, kd, vd = (to_device(x, "bf16") for x in (q, k, v))
    ref_o, ref_l = moba.prefill(qd, kd, vd, B, topk)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o, l = moba.prefill(qd, kd, vd, B, topk)
    s.synchronize()
    assert torch.equal(o.view(torch.int16), ref_o.view(torch.int16))
    assert torch.equal(l, ref_l)


# Decode step: (N, H, D, B, topk, seed). B dividing N or not (partial own
# block), the first token, D = 64, the own block alone, topk above the number
# of past blocks (full attention), many blocks with B = 64, B not a multiple
# of the attention chunk.
DECODE = [
    (4096, 4, 128, 256, 3, 1),
    (4000, 2, 128, 256, 3, 2),
    (1, 2, 128, 64, 3, 3),
    (777, 3, 64, 128, 2, 4),
    (2048, 2, 128, 512, 1, 5),
    (8192, 2, 128, 512, 100, 6),
    (6000, 1, 128, 64, 9, 7),
    (3333, 2, 128, 1000, 2, 8),
    (32768, 8, 128, 512, 3, 9),
    (140000, 1, 64, 64, 4, 10),      # 2187 past blocks: gate scores outside LDS
    (32768, 2, 128, 512, 16, 11),    # 8192 kept keys: the largest one-launch step
]


@pytest.mark.parametrize("case", DECODE, ids=lambda c: "N{}_H{}_D{}_B{}_k{}".format(*c[:5]))
def test_decode_parity(moba, case):
    from oracle import gate_scores, moba_decode_ref, pooled_keys_fp32
    from tests.parity import near_tie
    N, H, D, B, topk, seed = case
    q, k, v = synth.make_qkv(N, H, D, seed=[300 + seed, 0], dtype="bf16")
    qd, kd, vd = (to_device(x, "bf16") for x in (q, k, v))
    qn = qd[N - 1].contiguous()
    sel = torch.empty((H, topk), dtype=torch.int32, device="cuda")
    out, lse = moba.decode(qn, kd, vd, B, topk, sel=sel)
    j = (N - 1) // B
    # The same call with the block means supplied (as a decode loop would keep them).
    if j > 0:
        # Exact fp64 means rounded once to fp32, as moba_block_mean_keys writes them
        # (computed here with torch so that any block size works).
        kbar = kd[:j * B].double().reshape(j, B, H, D).mean(dim=1).float().permute(1, 0, 2).contiguous()
    else:
        kbar = None
    # With the means supplied, a gated step with few kept keys runs as one
    # launch (a different summation order): same selection, outputs to the bar.
    sel2 = torch.empty_like(sel)
    out2, lse2 = moba.decode(qn, kd, vd, B, topk, kbar=kbar, sel=sel2)
    torch.cuda.synchronize()
    assert torch.equal(sel, sel2)
    gsel = sel.cpu().numpy()
    _, _, rsel = moba_decode_ref(q[N - 1], k, v, B, topk)
    exempt = exempt_rowmax = 0
    for h in range(H):
        if np.array_equal(gsel[h], rsel[h]):
            continue
        # Only a ranked step (more past blocks than kept ones) may differ, with
        # the padding in place, and only on a near-tie of the fp32 gate scores.
        assert j >= topk and np.array_equal(gsel[h] == -1, rsel[h] == -1), (h, gsel[h], rsel[h])
        g = gate_scores(q[N - 1, h][None, :], pooled_keys_fp32(k[:j * B], B)[h])[0].astype(np.float64)
        b = [int(x) for x in gsel[h] if x >= 0]
        assert b == sorted(set(b)) and b[-1] == j and b[0] >= 0
        pair, rowmax = near_tie(g, [int(x) for x in rsel[h] if 0 <= x < j], b[:-1], j=j)
        assert pair, (h, gsel[h], rsel[h])
        exempt += 1
        exempt_rowmax += int(rowmax)
    ro, rl, _ = moba_decode_ref(q[N - 1], k, v, B, topk, sel=gsel)
    err_o = max(max_abs(out.float().cpu().numpy(), ro), max_abs(out2.float().cpu().numpy(), ro))
    err_l = max(max_abs(lse.cpu().numpy(), rl), max_abs(lse2.cpu().numpy(), rl))
    log(f"  decode N={N} H={H} D={D} B={B} k={topk}: exempt {exempt} (row-max rule {exempt_rowmax}), max|out| err {err_o:.3e}, max|lse| err {err_l:.3e}")
    assert err_o <= OUT_TOL["bf16"]
    assert err_l <= LSE_TOL["bf16"]


BACKWARD = [  # (N, H, D, B, topk, seed)
    (1024, 2, 128, 128, 3, 1),
    (512, 1, 64, 64, 2, 2),
    (2048, 2, 128, 512, 3, 3),
    (768, 2, 128, 256, 1, 4),        # own block only: no query lists
    (1024, 1, 128, 128, 16, 5),      # top_k > n: full causal attention
    (1536, 2, 64, 192, 4, 6),        # B not a multiple of 128 or 256
    (4096, 1, 128, 256, 5, 7),
    (1920, 2, 128, 320, 3, 8),       # D = 128, last 128-key chunk half empty, own tiles of 256 + 64 queries
]
# Gradients are compared with the fp64 oracle (same selection) relative to the
# largest |gradient| of each tensor (max-norm) and in relative L2: the GPU
# rounds P and dS to bf16 for the matrix cores, takes Δ from the bf16 forward
# output and returns bf16 (rounding alone gives a relative L2 of ~2.3e-3).
GRAD_REL_TOL = 1e-2
GRAD_L2_TOL = 5e-3


@pytest.mark.parametrize("case", BACKWARD, ids=lambda c: "N{}_H{}_D{}_B{}_k{}".format(*c[:5]))
def test_backward_parity(moba, case):
    from oracle import moba_backward_ref
    N, H, D, B, topk, seed = case
    q, k, v = synth.make_qkv(N, H, D, seed=[400 + seed, 0], dtype="bf16")
    do = synth.make_grad(N, H, D, seed=[400 + seed, 1])
    qd, kd, vd, dod = (to_device(x, "bf16") for x in (q, k, v, do))
    out, lse = moba.prefill(qd, kd, vd, B, topk)
    dq, dk, dv = moba.prefill_backward(qd, kd, vd, out, lse, dod, B, topk)
    sel = moba.gate_topk(qd, kd, B, topk)
    torch.cuda.synchronize()
    rq, rk, rv, _ = moba_backward_ref(q, k, v, do, B, topk, sel=sel.cpu().numpy())
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        g = got.float().cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(g)), name
        err = float(np.max(np.abs(g - ref)))
        scale = float(np.max(np.abs(ref)))
        rel = float(np.linalg.norm(g - ref) / max(np.linalg.norm(ref), 1e-30))
        log(f"  backward N={N} H={H} D={D} B={B} k={topk} {name}: max|err| {err:.3e} (max|ref| {scale:.3e}), "
            f"rel L2 {rel:.3e}")
        assert err <= GRAD_REL_TOL * scale, name
        assert rel <= GRAD_L2_TOL, name
    # Deterministic: a second call gives the same bits.
    dq2, dk2, dv2 = moba.prefill_backward(qd, kd, vd, out, lse, dod, B, topk)
    torch.cuda.synchronize()
    for a_, b_ in ((dq, dq2), (dk, dk2), (dv, dv2)):
        assert torch.equal(a_.view(torch.int16), b_.view(torch.int16))


def test_backward_h32_one_head(moba):
    """The h32 workload (N=32768, 32 heads, B=512, top-3) at full size; head 5's
    gradients (every row) against the oracle's per-block evaluation."""
    from oracle import moba_backward_ref
    w, q, k, v = synth.make_workload("h32")
    do = synth.make_grad(w.N, w.H, w.D, seed=[402, 9])
    qd, kd, vd, dod = (to_device(x, "bf16") for x in (q, k, v, do))
    out, lse = moba.prefill(qd, kd, vd, w.block_size, w.topk)
    dq, dk, dv = moba.prefill_backward(qd, kd, vd, out, lse, dod, w.block_size, w.topk)
    sel = moba.gate_topk(qd, kd, w.block_size, w.topk)
    torch.cuda.synchronize()
    h = 5
    rq, rk, rv, _ = moba_backward_ref(q, k, v, do, w.block_size, w.topk, sel=sel.cpu().numpy(), heads=[h],
                                      method="blocks")
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        g = got[:, h].float().cpu().numpy().astype(np.float64)
        r = ref[:, 0]
        err = float(np.max(np.abs(g - r)))
        scale = float(np.max(np.abs(r)))
        rel = float(np.linalg.norm(g - r) / np.linalg.norm(r))
        log(f"  backward h32 head {h} {name}: max|err| {err:.3e} (max|ref| {scale:.3e}), rel L2 {rel:.3e}")
        assert err <= GRAD_REL_TOL * scale and rel <= GRAD_L2_TOL, name


POOLED = [  # (N, H, D, B, topk, pooling, seed)
    (2048, 2, 128, 128, 3, "max", 1),
    (2048, 2, 128, 128, 3, "weighted", 2),
    (4096, 1, 64, 256, 4, "max", 3),
    (4096, 2, 64, 256, 2, "weighted", 4),
]


@pytest.mark.parametrize("case", POOLED, ids=lambda c: "N{}_H{}_D{}_B{}_k{}_{}".format(*c[:6]))
def test_pooling_variants(moba, case):
    from oracle import moba_ref, pooled_keys_fp32, select_blocks
    N, H, D, B, topk, pooling, seed = case
    q, k, v = synth.make_qkv(N, H, D, seed=[500 + seed, 0], dtype="bf16")
    w = np.random.default_rng([500 + seed, 1]).uniform(0.0, 1.0, (H, N)).astype(np.float32) \
        if pooling == "weighted" else None
    qd, kd, vd = (to_device(x, "bf16") for x in (q, k, v))
    wd = torch.from_numpy(w).cuda() if w is not None else None
    kbar = moba.block_pool_keys(kd, B, pooling, wd)
    sel = moba.gate_topk_pooled(qd, kd, B, topk, pooling, wd)
    out, lse = moba.prefill_pooled(qd, kd, vd, B, topk, pooling, wd)
    torch.cuda.synchronize()
    ref_kbar = pooled_keys_fp32(k, B, pooling, w)
    kb = kbar.cpu().numpy()
    if pooling == "max":
        assert np.array_equal(kb, ref_kbar)
    else:   # fp64 sums in another order: at most one fp32 rounding step apart
        assert np.all(np.abs(kb - ref_kbar) <= np.spacing(np.abs(ref_kbar)))
    gsel = sel.cpu().numpy()
    ref_sel, _ = select_blocks(q, k, B, topk, pooling=pooling, weights=w)
    cmp = compare_selection(gsel, ref_sel, q, k, B, topk, pooling=pooling, weights=w)
    assert not cmp["bad"], cmp["bad"][:5]
    ref_out, ref_lse, _ = moba_ref(q, k, v, B, topk, sel=gsel)
    e_out = max_abs(out.float().cpu().numpy(), ref_out)
    e_lse = max_abs(lse.cpu().numpy(), ref_lse)
    log(f"  pooling {pooling} N={N} H={H} D={D} B={B} k={topk}: sel mismatch {cmp['mismatch']} "
        f"(exempt {cmp['exempt']}, row-max rule {cmp['exempt_rowmax']}), max|out| err {e_out:.3e}, max|lse| err {e_lse:.3e}")
    assert e_out <= OUT_TOL["bf16"] and e_lse <= LSE_TOL["bf16"]
    # The mean pooling differs from max pooling on these inputs: the selections are not all equal.
    if pooling == "max":
        assert not np.array_equal(gsel, moba.gate_topk(qd, kd, B, topk).cpu().numpy())


@pytest.mark.parametrize("pooling", ["max", "weighted"])
def test_backward_pooled(moba, pooling):
    """The backward pass recomputes the selection with the same pooling."""
    from oracle import moba_backward_ref
    N, H, D, B, topk = 1024, 2, 128, 128, 3
    q, k, v = synth.make_qkv(N, H, D, seed=[510, 0], dtype="bf16")
    do = synth.make_grad(N, H, D, seed=[510, 1])
    w = np.random.default_rng([510, 2]).uniform(0.0, 1.0, (H, N)).astype(np.float32) \
        if pooling == "weighted" else None
    qd, kd, vd, dod = (to_device(x, "bf16") for x in (q, k, v, do))
    wd = torch.from_numpy(w).cuda() if w is not None else None
    out, lse = moba.prefill_pooled(qd, kd, vd, B, topk, pooling, wd)
    dq, dk, dv = moba.prefill_backward(qd, kd, vd, out, lse, dod, B, topk, pooling=pooling, weights=wd)
    sel = moba.gate_topk_pooled(qd, kd, B, topk, pooling, wd)
    torch.cuda.synchronize()
    rq, rk, rv, _ = moba_backward_ref(q, k, v, do, B, topk, sel=sel.cpu().numpy())
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        g = got.float().cpu().numpy().astype(np.float64)
        rel = float(np.linalg.norm(g - ref) / np.linalg.norm(ref))
        log(f"  backward {pooling}-pooled {name}: rel L2 {rel:.3e}")
        assert rel <= GRAD_L2_TOL and float(np.max(np.abs(g - ref))) <= GRAD_REL_TOL * float(np.max(np.abs(ref)))


def test_dense_path(moba):
    """top_k >= n keeps every block: the call runs as causal attention over one
    block of N tokens. Sampled rows against the oracle; top_k = n and n + 8 give
    the same bits; the backward against the oracle on a smaller case."""
    from oracle import moba_backward_ref, moba_ref
    N, H, D, B = 16384, 2, 128, 512
    n = N // B
    q, k, v = synth.make_qkv(N, H, D, seed=[520, 0], dtype="bf16")
    qd, kd, vd = (to_device(x, "bf16") for x in (q, k, v))
    out, lse = moba.prefill(qd, kd, vd, B, n)
    out2, lse2 = moba.prefill(qd, kd, vd, B, n + 8)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), lse2.view(torch.int32))
    rows = synth.sample_rows(N, 2048, 521)
    ref_out, ref_lse, _ = moba_ref(q, k, v, B, n, rows=rows)
    e_out = max_abs(out.float().cpu().numpy()[rows], ref_out)
    e_lse = max_abs(lse.cpu().numpy()[:, rows], ref_lse)
    log(f"  dense N={N} H={H} top-k {n}: max|out| err {e_out:.3e}, max|lse| err {e_lse:.3e}")
    assert e_out <= OUT_TOL["bf16"] and e_lse <= LSE_TOL["bf16"]

    N, H, D, B = 2048, 2, 64, 256
    q, k, v = synth.make_qkv(N, H, D, seed=[522, 0], dtype="bf16")
    do = synth.make_grad(N, H, D, seed=[522, 1])
    qd, kd, vd, dod = (to_device(x, "bf16") for x in (q, k, v, do))
    out, lse = moba.prefill(qd, kd, vd, B, N // B)
    dq, dk, dv = moba.prefill_backward(qd, kd, vd, out, lse, dod, B, N // B)
    torch.cuda.synchronize()
    rq, rk, rv, _ = moba_backward_ref(q, k, v, do, B, N // B)
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        g = got.float().cpu().numpy().astype(np.float64)
        rel = float(np.linalg.norm(g - ref) / np.linalg.norm(ref))
        log(f"  dense backward {name}: rel L2 {rel:.3e}")
        assert rel <= GRAD_L2_TOL and float(np.max(np.abs(g - ref))) <= GRAD_REL_TOL * float(np.max(np.abs(ref)))


VARLEN = [  # (cu_seqlens, H, D, B, topk, seed)
    ([0, 1024, 1536, 4096], 2, 128, 128, 3, 1),
    ([0, 512, 512, 2560, 2816], 1, 64, 256, 4, 2),     # an empty sequence, a one-block sequence
    ([0, 4096, 8192], 2, 128, 512, 3, 3),
    ([0, 192, 448, 1728], 2, 128, 64, 20, 4),           # 19 past blocks kept: the separate merge
    ([0, 192, 448, 1728], 1, 64, 64, 45, 5),            # topk above the longest sequence's 20 blocks
]


@pytest.mark.parametrize("case", VARLEN, ids=lambda c: "S{}_T{}_H{}_D{}_B{}_k{}".format(len(c[0]) - 1, c[0][-1],
                                                                                       *c[1:5]))
def test_varlen_parity(moba, case):
    """Packed sequences: selections, outputs and gradients against the oracle
    (each sequence on its own), and every sequence equal to a separate call."""
    from oracle import moba_backward_ref_varlen, moba_ref_varlen
    cu, H, D, B, topk, seed = case
    T = cu[-1]
    q, k, v = synth.make_qkv(T, H, D, seed=[530 + seed, 0], dtype="bf16")
    do = synth.make_grad(T, H, D, seed=[530 + seed, 1])
    qd, kd, vd, dod = (to_device(x, "bf16") for x in (q, k, v, do))
    sel = moba.gate_topk_varlen(qd, kd, cu, B, topk)
    out, lse = moba.prefill_varlen(qd, kd, vd, cu, B, topk)
    dq, dk, dv = moba.prefill_backward_varlen(qd, kd, vd, out, lse, dod, cu, B, topk)
    torch.cuda.synchronize()
    gsel = sel.cpu().numpy()
    ref_out, ref_lse, ref_sel = moba_ref_varlen(q, k, v, cu, B, topk)
    mism = int(np.sum((gsel != ref_sel).any(axis=-1)))
    # Any selection difference must be a near-tie inside one sequence; these seeds have none.
    assert mism == 0, mism
    e_out = max_abs(out.float().cpu().numpy(), ref_out)
    e_lse = max_abs(lse.cpu().numpy(), ref_lse)
    rq, rk, rv = moba_backward_ref_varlen(q, k, v, do, cu, B, topk, sel=gsel)
    rels = []
    for got, ref in ((dq, rq), (dk, rk), (dv, rv)):
        g = got.float().cpu().numpy().astype(np.float64)
        rels.append(float(np.linalg.norm(g - ref) / np.linalg.norm(ref)))
        assert float(np.max(np.abs(g - ref))) <= GRAD_REL_TOL * float(np.max(np.abs(ref)))
    log(f"  varlen cu={cu} H={H} D={D} B={B} k={topk}: max|out| err {e_out:.3e}, max|lse| err {e_lse:.3e}, "
        f"grad rel L2 {max(rels):.3e}")
    assert e_out <= OUT_TOL["bf16"] and e_lse <= LSE_TOL["bf16"] and max(rels) <= GRAD_L2_TOL
    # Each sequence equals a separate single-sequence call (the dense path too when it applies).
    for a, b in zip(cu[:-1], cu[1:]):
        if b == a:
            continue
        o1, l1 = moba.prefill(qd[a:b].contiguous(), kd[a:b].contiguous(), vd[a:b].contiguous(), B, topk)
        torch.cuda.synchronize()
        err = float((o1.float() - out[a:b].float()).abs().max())
        assert err <= 2 * OUT_TOL["bf16"], (a, b, err)


def test_largest_block_count(moba):
    """n = 4096 blocks (the largest supported) with top-32 (the widest ranked
    list): the gate reads the split means from L2 and keeps one bitmap buffer,
    every query keeps 31 past blocks (the separate merge). Sampled rows."""
    from oracle import moba_ref, select_blocks
    N, H, D, B, topk = 262144, 1, 64, 64, 32
    q, k, v = synth.make_qkv(N, H, D, seed=[540, 0], dtype="bf16")
    qd, kd, vd = (to_device(x, "bf16") for x in (q, k, v))
    sel = moba.gate_topk(qd, kd, B, topk)
    out, lse = moba.prefill(qd, kd, vd, B, topk)
    torch.cuda.synchronize()
    rows = synth.sample_rows(N, 1024, 541)
    gsel = sel.cpu().numpy()[:, rows]
    ref_sel, _ = select_blocks(q, k, B, topk, rows=rows)
    cmp = compare_selection(gsel, ref_sel, q, k, B, topk, rows=rows)
    assert not cmp["bad"], cmp["bad"][:3]
    ref_out, ref_lse, _ = moba_ref(q, k, v, B, topk, sel=gsel, rows=rows, method="blocks")
    e_out = max_abs(out.float().cpu().numpy()[rows], ref_out)
    e_lse = max_abs(lse.cpu().numpy()[:, rows], ref_lse)
    log(f"  n=4096 top-32: sel mismatch {cmp['mismatch']} (exempt {cmp['exempt']}, row-max rule {cmp['exempt_rowmax']}), max|out| err {e_out:.3e}, "
        f"max|lse| err {e_lse:.3e}")
    assert e_out <= OUT_TOL["bf16"] and e_lse <= LSE_TOL["bf16"]


def test_poisoned_workspace(moba):
    """Every workspace byte set to 0xFF (NaN in fp32/bf16, -1 in int32) before
    the stages: the results stay finite and bitwise equal to an ordinary call,
    so no stage reads workspace memory that an earlier stage of the same call
    did not write (the regrouped query lists, the work items, the partial
    outputs). h32-shaped prefill, a packed batch through the separate merge,
    the backward, and an unfused decode step."""
    def same(a, b):
        return torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))

    cases = []
    w, q, k, v = synth.make_workload("h32")
    qd, kd, vd = (to_device(x, "bf16") for x in (q, k, v))
    del q, k, v
    cases.append(("h32 prefill", lambda: moba.prefill(qd, kd, vd, w.block_size, w.topk)))
    cu = [0, 192, 448, 1728]
    q2, k2, v2 = synth.make_qkv(1728, 2, 128, seed=[560, 0], dtype="bf16")
    q2d, k2d, v2d = (to_device(x, "bf16") for x in (q2, k2, v2))
    cases.append(("varlen prefill", lambda: moba.prefill_varlen(q2d, k2d, v2d, cu, 64, 20)))
    q3, k3, v3 = synth.make_qkv(2048, 2, 128, seed=[561, 0], dtype="bf16")
    do3 = synth.make_grad(2048, 2, 128, seed=[561, 1])
    q3d, k3d, v3d, do3d = (to_device(x, "bf16") for x in (q3, k3, v3, do3))
    o3, l3 = moba.prefill(q3d, k3d, v3d, 256, 3)
    cases.append(("backward", lambda: moba.prefill_backward(q3d, k3d, v3d, o3, l3, do3d, 256, 3)))
    cases.append(("decode", lambda: moba.decode(q3d[2047].contiguous(), k3d, v3d, 64, 40)))
    try:
        for name, fn in cases:
            log(f"  poisoned workspace: {name}")
            moba.debug_poison_workspace(False)
            ref = fn()
            moba.debug_poison_workspace(True)
            got = fn()
            moba.debug_poison_workspace(False)
            torch.cuda.synchronize()
            for r, g in zip(ref, got):
                assert bool(torch.isfinite(g.float()).all()), name
                assert same(r, g), name
    finally:
        moba.debug_poison_workspace(False)
