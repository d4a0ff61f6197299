"""GPU test of the allocation-free decode entry point (moba_decode_fwd_noalloc):
through the C-ABI, its results equal moba_decode_fwd's bit for bit, on two calls
in a row (the second with a smaller input, so that it runs on scratch memory the
first one left behind), and a step whose workspace exceeds the scratch array is
refused with MOBA_ERR_UNSUPPORTED, its outputs untouched."""

import ctypes

import numpy as np
import pytest

from block_sparse_long_gating_amd import synth
from tests.parity import OUT_TOL, log, max_abs, to_device

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moba():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import block_sparse_long_gating_amd as m
    m.load_library()
    return m


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


# (N, H, D, B, topk, kbar supplied, seed): full attention over a 32K x 8-head
# cache (split path, the larger workspace), then a gated step over a smaller
# cache that pools its own block means into the scratch memory; then the same
# pair in the other order.
CALLS = [
    (32768, 8, 128, 512, 100, False, 1),
    (4000, 2, 128, 256, 3, False, 2),
    (6000, 1, 64, 64, 9, False, 3),
]


def _run_pair(moba, first, second):
    from oracle import moba_decode_ref
    for N, H, D, B, topk, with_kbar, seed in (first, second):
        q, k, v = synth.make_qkv(N, H, D, seed=[700 + seed, 0], dtype="bf16")
        qd, kd, vd = (to_device(x, "bf16") for x in (q, k, v))
        qn = qd[N - 1].contiguous()
        j = (N - 1) // B
        kbar = moba.block_mean_keys(kd[:j * B].contiguous(), B) if (with_kbar and j > 0) else None
        sel_a = torch.full((H, topk), -7, dtype=torch.int32, device="cuda")
        sel_b = torch.full((H, topk), -7, dtype=torch.int32, device="cuda")
        log(f"  noalloc decode N={N} H={H} D={D} B={B} topk={topk}")
        out_a, lse_a = moba.decode(qn, kd, vd, B, topk, kbar=kbar, sel=sel_a)
        out_b, lse_b = moba.decode(qn, kd, vd, B, topk, kbar=kbar, sel=sel_b, noalloc=True)
        torch.cuda.synchronize()
        assert torch.equal(_bits(out_a), _bits(out_b))
        assert torch.equal(_bits(lse_a), _bits(lse_b))
        assert torch.equal(sel_a, sel_b)
        ro, rl, _ = moba_decode_ref(q[N - 1], k, v, B, topk, sel=sel_a.cpu().numpy())
        err = max_abs(out_b.float().cpu().numpy(), ro)
        log(f"    bitwise equal to moba_decode_fwd; max|out - oracle| {err:.3e}")
        assert err <= OUT_TOL["bf16"]


def test_noalloc_matches_pooled_entry_point(moba):
    _run_pair(moba, CALLS[0], CALLS[1])
    _run_pair(moba, CALLS[2], CALLS[1])


def test_noalloc_refuses_oversized_workspace(moba):
    """Full attention over a 1M-token, 32-head cache of 64-key blocks needs
    ~140 MB of partials (16384 units per head): refused before any work, the
    outputs untouched."""
    lib = moba.load_library()
    N, H, D, B = 1 << 20, 32, 64, 64
    k = torch.zeros((N, H, D), dtype=torch.bfloat16, device="cuda")
    q = torch.zeros((H, D), dtype=torch.bfloat16, device="cuda")
    out = torch.full((H, D), 3.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((H,), 5.0, dtype=torch.float32, device="cuda")
    st = lib.moba_decode_fwd_noalloc(q.data_ptr(), k.data_ptr(), k.data_ptr(), None, 0, out.data_ptr(),
                                     lse.data_ptr(), None, N, H, D, B, 1 << 20, None)
    assert st == 2, st
    torch.cuda.synchronize()
    assert bool((out == 3.0).all()) and bool((lse == 5.0).all())
