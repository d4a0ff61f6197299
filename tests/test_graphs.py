"""The library's calls and HIP graph capture.

Calls that take workspace from the library's stream-ordered pool refuse a
stream under capture (MOBA_ERR_UNSUPPORTED, nothing enqueued); that refusal is
tested here.

The replay tests below record calls into a graph and check every replay bit
for bit against an eager call on the same inputs; between replays they run
their own eager work (new input values copied into the captured tensors, the
outputs overwritten with a fill kernel) and synchronise, and the new input
values change the selections, the lengths of the per-block query lists and the
number of attention work items from one replay to the next. They are skipped:
the prefill replay, recorded with its pool allocation and free as graph memory
nodes, ended in a GPU memory fault, and no cause in this library has been
shown, so no replay is run until one is.
"""
import pytest

torch = pytest.importorskip("torch")

from block_sparse_long_gating_amd import synth  # noqa: E402
from tests.parity import log, to_device  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moba():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import block_sparse_long_gating_amd as m
    m.load_library()
    return m


def _inputs(N, H, D, seed):
    return [to_device(x, "bf16") for x in synth.make_qkv(N, H, D, seed=seed, dtype="bf16")]


def _capture(fn):
    """Warm up fn on a side stream, then record it into a graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


REPLAY_SKIP = ("graph replay not run: a prefill recorded with its pool allocation faulted the GPU on replay and no "
               "cause in this library has been shown; allocating calls now refuse capture")


def _same(a, b):
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a, b)


@pytest.mark.skip(reason=REPLAY_SKIP)
def test_prefill_graph(moba):
    N, H, D, B, topk = 4096, 2, 128, 256, 3
    q, k, v = _inputs(N, H, D, [700, 0])
    out = torch.empty_like(q)
    lse = torch.empty((H, N), dtype=torch.float32, device=q.device)
    g = _capture(lambda: moba.prefill(q, k, v, B, topk, out=out, lse=lse))
    items = []
    for r in range(4):
        nq, nk, nv = _inputs(N, H, D, [700, r])
        q.copy_(nq)
        k.copy_(nk)
        v.copy_(nv)
        ref_o, ref_l = moba.prefill(q, k, v, B, topk)
        sel = moba.gate_topk(q, k, B, topk)
        items.append(int((sel[:, :, :-1] >= 0).sum().item()))
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert _same(out, ref_o), f"replay {r}: out differs from the eager call"
        assert _same(lse, ref_l), f"replay {r}: lse differs from the eager call"
    log(f"prefill graph: 4 replays bitwise equal to eager; past selections per replay {items}")


@pytest.mark.skip(reason=REPLAY_SKIP)
def test_backward_graph(moba):
    N, H, D, B, topk = 2048, 2, 128, 256, 3
    q, k, v = _inputs(N, H, D, [710, 0])
    do = _inputs(N, H, D, [711, 0])[0]
    out, lse = moba.prefill(q, k, v, B, topk)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    g = _capture(lambda: moba.prefill_backward(q, k, v, out, lse, do, B, topk, dq=dq, dk=dk, dv=dv))
    for r in range(3):
        nq, nk, nv = _inputs(N, H, D, [710, r])
        q.copy_(nq)
        k.copy_(nk)
        v.copy_(nv)
        o2, l2 = moba.prefill(q, k, v, B, topk)
        out.copy_(o2)
        lse.copy_(l2)
        rq, rk, rv = moba.prefill_backward(q, k, v, out, lse, do, B, topk)
        for t in (dq, dk, dv):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert _same(dq, rq) and _same(dk, rk) and _same(dv, rv), f"replay {r}: gradients differ"
    log("backward graph: 3 replays bitwise equal to eager")


@pytest.mark.skip(reason=REPLAY_SKIP)
@pytest.mark.parametrize("noalloc", [False, True], ids=["pooled", "noalloc"])
def test_decode_graph(moba, noalloc):
    N, H, D, B, topk = 8192, 4, 128, 512, 3
    q, k, v = _inputs(N, H, D, [720, 0])
    qn = q[N - 1].contiguous()
    out = torch.empty_like(qn)
    lse = torch.empty((H,), dtype=torch.float32, device=q.device)
    g = _capture(lambda: moba.decode(qn, k, v, B, topk, out=out, lse=lse, noalloc=noalloc))
    for r in range(4):
        nq, nk, nv = _inputs(N, H, D, [720, r])
        qn.copy_(nq[N - 1])
        k.copy_(nk)
        v.copy_(nv)
        ref_o, ref_l = moba.decode(qn, k, v, B, topk)
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert _same(out, ref_o) and _same(lse, ref_l), f"replay {r}: decode differs from the eager call"
    log(f"decode graph ({'noalloc' if noalloc else 'pooled'}): 4 replays bitwise equal to eager")


@pytest.mark.filterwarnings("ignore:The CUDA Graph is empty")
@pytest.mark.parametrize("call", ["prefill", "backward", "gate_lists"])
def test_allocating_calls_refuse_capture(moba, call):
    """Under capture an allocating call returns MOBA_ERR_UNSUPPORTED before
    enqueuing anything; the stream and the library work eagerly afterwards."""
    N, H, D, B, topk = 2048, 2, 128, 256, 3
    q, k, v = _inputs(N, H, D, [730, 0])
    ref_o, ref_l = moba.prefill(q, k, v, B, topk)
    out = torch.empty_like(q)
    lse = torch.empty((H, N), dtype=torch.float32, device=q.device)
    do = torch.ones_like(q)
    torch.cuda.synchronize()
    calls = {
        "prefill": lambda: moba.prefill(q, k, v, B, topk, out=out, lse=lse),
        "backward": lambda: moba.prefill_backward(q, k, v, ref_o, ref_l, do, B, topk),
        "gate_lists": lambda: moba.block_query_lists(q, k, B, topk),
    }
    g = torch.cuda.CUDAGraph()
    with pytest.raises(moba.MobaError) as err:
        with torch.cuda.graph(g):
            calls[call]()
    assert err.value.status == 2, str(err.value)
    del g
    torch.cuda.synchronize()
    o, l = moba.prefill(q, k, v, B, topk)
    torch.cuda.synchronize()
    assert _same(o, ref_o) and _same(l, ref_l)
    log(f"{call}: refused under capture ({err.value}); eager calls unaffected")
