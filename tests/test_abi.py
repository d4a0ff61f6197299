"""CPU tests of the C-ABI boundary: the library loads, exports every declared
symbol, and rejects bad arguments before touching the GPU."""

import ctypes
import os
import re

import pytest

import block_sparse_long_gating_amd as moba

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moba.h")

OK, INVALID, UNSUPPORTED = 0, 1, 2


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moba_\w+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(moba.library_path()):
        pytest.fail("libmoba.so is not built (run __graft_entry__.build())")
    return moba.load_library()


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("moba_gate_topk", "moba_prefill_fwd", "moba_gate_topk_f32", "moba_prefill_fwd_f32",
              "moba_block_mean_keys", "moba_block_mean_keys_f32", "moba_status_string", "moba_last_hip_error"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    raw = ctypes.CDLL(moba.library_path())
    for name in declared_functions():
        assert hasattr(raw, name), f"{name} declared in moba.h but not exported"


def test_binding_covers_every_symbol():
    assert set(declared_functions()) == set(moba._SIGNATURES)


def test_header_constants_match_binding():
    src = open(HEADER).read()
    assert int(re.search(r"#define MOBA_MAX_TOPK (\d+)", src).group(1)) == moba.MAX_TOPK
    assert int(re.search(r"#define MOBA_MAX_BLOCKS (\d+)", src).group(1)) == moba.MAX_BLOCKS
    for code, name in moba.STATUS.items():
        assert re.search(rf"{name} = {code}\b", src)


def test_status_strings(lib):
    for code, name in moba.STATUS.items():
        assert lib.moba_status_string(code).decode() == name
    assert lib.moba_status_string(99).decode() == "MOBA_ERR_UNKNOWN"
    assert lib.moba_last_hip_error() == 0


def test_poison_switch_is_host_state(lib):
    """The workspace-poisoning switch only flips host state and returns the
    previous setting (no GPU needed)."""
    assert lib.moba_debug_poison_workspace(1) == 0
    assert lib.moba_debug_poison_workspace(7) == 1
    assert lib.moba_debug_poison_workspace(0) == 1
    assert lib.moba_debug_poison_workspace(0) == 0


# Fake, never dereferenced, 16-byte aligned addresses: every call below must be
# rejected by the host-side checks before any HIP call.
A = 0x10000


def prefill(lib, N=1024, H=1, D=128, B=128, topk=3, ptrs=(A, A, A, A, A), f32=False):
    fn = lib.moba_prefill_fwd_f32 if f32 else lib.moba_prefill_fwd
    return fn(*ptrs, N, H, D, B, topk, None)


def gate(lib, N=1024, H=1, D=128, B=128, topk=3, ptrs=(A, A, A), f32=False):
    fn = lib.moba_gate_topk_f32 if f32 else lib.moba_gate_topk
    return fn(*ptrs, N, H, D, B, topk, None)


def pool(lib, N=1024, H=1, D=128, B=128, ptrs=(A, A), f32=False):
    fn = lib.moba_block_mean_keys_f32 if f32 else lib.moba_block_mean_keys
    return fn(*ptrs, N, H, D, B, None)


@pytest.mark.parametrize("f32", [False, True])
def test_null_pointers(lib, f32):
    for i in range(5):
        ptrs = [A] * 5
        ptrs[i] = None
        assert prefill(lib, ptrs=tuple(ptrs), f32=f32) == INVALID
    for i in range(3):
        ptrs = [A] * 3
        ptrs[i] = None
        assert gate(lib, ptrs=tuple(ptrs), f32=f32) == INVALID
    assert pool(lib, ptrs=(None, A), f32=f32) == INVALID
    assert pool(lib, ptrs=(A, None), f32=f32) == INVALID


@pytest.mark.parametrize("f32", [False, True])
def test_invalid_shapes(lib, f32):
    for kw in (dict(N=0), dict(N=-5), dict(H=0), dict(topk=0), dict(topk=-1), dict(B=0),
               dict(N=1000, B=128), dict(N=1024, B=384)):
        assert prefill(lib, f32=f32, **kw) == INVALID, kw
        assert gate(lib, f32=f32, **kw) == INVALID, kw
    assert pool(lib, N=1000, B=128, f32=f32) == INVALID


@pytest.mark.parametrize("f32", [False, True])
def test_unsupported_shapes(lib, f32):
    for kw in (dict(D=96), dict(D=256), dict(D=32), dict(N=960, B=96), dict(N=1 << 28, B=1 << 16),
               dict(N=64 * 5000, B=64), dict(N=64 * 100, B=64, topk=33), dict(H=70000)):
        assert prefill(lib, f32=f32, **kw) == UNSUPPORTED, kw
        assert gate(lib, f32=f32, **kw) == UNSUPPORTED, kw
    for i in range(5):
        ptrs = [A] * 5
        ptrs[i] = A + 4
        assert prefill(lib, ptrs=tuple(ptrs), f32=f32) == UNSUPPORTED
    assert gate(lib, ptrs=(A, A, A + 8), f32=f32) == UNSUPPORTED
    assert pool(lib, D=80, f32=f32) == UNSUPPORTED


def test_topk_at_least_n_is_not_limited(lib):
    # n = 100 blocks, topk >= n selects everything and is accepted by the checks
    # (it then needs a device, which this test does not reach: an invalid H stops it)
    assert prefill(lib, N=6400, B=64, topk=150, H=0) == INVALID
    assert prefill(lib, N=6400, B=64, topk=50) == UNSUPPORTED


def test_python_binding_rejects_bad_tensors():
    import torch
    q = torch.zeros(64, 1, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        moba.prefill(q, q, q, 64, 3)          # not on a GPU
    with pytest.raises(TypeError):
        moba.prefill(q.half(), q.half(), q.half(), 64, 3)
    with pytest.raises(ValueError):
        moba.gate_topk(q[0], q[0], 64, 3)


def decode(lib, N=1000, H=2, D=128, B=128, topk=3, ptrs=(A, A, A, A, A), kbar=None, nb=0, sel=None):
    q, k, v, out, lse = ptrs
    return lib.moba_decode_fwd(q, k, v, kbar, nb, out, lse, sel, N, H, D, B, topk, None)


def test_decode_argument_checks(lib):
    for i in range(5):
        ptrs = [A] * 5
        ptrs[i] = None
        assert decode(lib, ptrs=tuple(ptrs)) == INVALID
    for kw in (dict(N=0), dict(H=0), dict(B=0), dict(topk=0), dict(topk=-2)):
        assert decode(lib, **kw) == INVALID, kw
    # kbar given with fewer blocks than the token's complete past blocks (999 // 128 = 7)
    assert decode(lib, kbar=A, nb=6) == INVALID
    for kw in (dict(D=96), dict(D=32), dict(H=70000), dict(N=128 * 100, topk=40)):
        assert decode(lib, **kw) == UNSUPPORTED, kw
    assert decode(lib, sel=A, topk=5000, N=128) == UNSUPPORTED
    for i in range(5):
        ptrs = [A] * 5
        ptrs[i] = A + 4
        assert decode(lib, ptrs=tuple(ptrs)) == UNSUPPORTED
    assert decode(lib, kbar=A + 4, nb=7) == UNSUPPORTED
    assert decode(lib, sel=A + 8) == UNSUPPORTED


def backward(lib, N=1024, H=2, D=128, B=128, topk=3, ptrs=(A,) * 9):
    q, k, v, out, lse, dout, dq, dk, dv = ptrs
    return lib.moba_prefill_bwd(q, k, v, out, lse, dout, dq, dk, dv, N, H, D, B, topk, None)


def test_backward_argument_checks(lib):
    for i in range(9):
        ptrs = [A] * 9
        ptrs[i] = None
        assert backward(lib, ptrs=tuple(ptrs)) == INVALID, i
    for kw in (dict(N=0), dict(H=0), dict(B=0), dict(topk=0), dict(N=1000)):
        assert backward(lib, **kw) == INVALID, kw
    for kw in (dict(D=96), dict(B=96, N=960), dict(H=70000), dict(N=128 * 100, topk=40)):
        assert backward(lib, **kw) == UNSUPPORTED, kw
    for i in range(9):
        ptrs = [A] * 9
        ptrs[i] = A + 4
        assert backward(lib, ptrs=tuple(ptrs)) == UNSUPPORTED, i


def test_query_lists_argument_checks(lib):
    """moba_block_query_lists: the same shape checks as the gate, plus the
    qidx capacity (the number of (query, past block) pairs, a closed form)."""
    def lists(N=1024, H=2, D=128, B=128, topk=3, ptrs=(A, A, A, A, A), qidx_len=None):
        n = N // B if B > 0 and N % B == 0 else 0
        pairs = H * sum(B * min(topk - 1, j) for j in range(n))
        return lib.moba_block_query_lists(*ptrs, pairs if qidx_len is None else qidx_len, N, H, D, B, topk, None)
    for i in range(5):
        ptrs = [A] * 5
        ptrs[i] = None
        assert lists(ptrs=tuple(ptrs)) == INVALID
        ptrs[i] = A + 4
        assert lists(ptrs=tuple(ptrs)) == UNSUPPORTED
    for kw in (dict(N=0), dict(H=0), dict(topk=0), dict(B=0), dict(N=1000, B=128)):
        assert lists(**kw) == INVALID, kw
    for kw in (dict(D=96), dict(N=960, B=96), dict(N=64 * 100, B=64, topk=33)):
        assert lists(**kw) == UNSUPPORTED, kw
    # 1024 tokens, 8 blocks of 128, top-3: 2 * 128 * (0 + 1 + 2 * 6) = 3328 pairs.
    assert lists(qidx_len=3327) == INVALID
    assert lists(topk=1, qidx_len=-1) == INVALID


def test_topk_for_sparsity_matches_oracle(lib):
    """Host-only helper (no GPU work): the library's dynamic k equals the oracle's."""
    from oracle import topk_for_sparsity
    lib.moba_topk_for_sparsity.restype = ctypes.c_int32
    lib.moba_topk_for_sparsity.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_double]
    for N, B in [(32768, 512), (131072, 2048), (262144, 4096), (1048576, 4096), (4096, 64), (512, 512)]:
        for s in (0.0, 0.5, 0.9, 0.906, 0.953, 0.99, 0.999):
            assert lib.moba_topk_for_sparsity(N, B, s) == topk_for_sparsity(N, B, s), (N, B, s)
    for args in ((0, 512, 0.9), (1000, 512, 0.9), (4096, 0, 0.9), (4096, 512, 1.0), (4096, 512, -0.1)):
        assert lib.moba_topk_for_sparsity(*args) == -INVALID, args


def test_pooled_argument_checks(lib):
    f = lib.moba_gate_topk_pooled
    assert f(A, A, None, A, 1024, 2, 128, 128, 3, 3, None) == INVALID          # unknown pooling
    assert f(A, A, None, A, 1024, 2, 128, 128, 3, 2, None) == INVALID          # weighted without weights
    assert f(A, A, A + 2, A, 1024, 2, 128, 128, 3, 2, None) == UNSUPPORTED     # misaligned weights
    assert lib.moba_block_pool_keys(A, None, A, 1024, 2, 128, 128, -1, None) == INVALID
    assert lib.moba_prefill_fwd_pooled(A, A, A, None, A, A, 1024, 2, 128, 128, 3, 2, None) == INVALID
    assert lib.moba_prefill_bwd_pooled(A, A, A, None, A, A, A, A, A, A, 1024, 2, 128, 128, 3, 7, None) == INVALID


def test_varlen_argument_checks(lib):
    def cu(*xs):
        arr = (ctypes.c_int64 * len(xs))(*xs)
        return arr

    g = lib.moba_prefill_fwd_varlen
    ok = cu(0, 256, 512)
    assert g(A, A, A, A, A, None, 2, 2, 128, 128, 3, None) == INVALID            # no cu_seqlens
    assert g(A, A, A, A, A, ok, 0, 2, 128, 128, 3, None) == INVALID              # no sequences
    assert g(A, A, A, A, A, cu(1, 257, 513), 2, 2, 128, 128, 3, None) == INVALID  # not starting at 0
    assert g(A, A, A, A, A, cu(0, 300, 512), 2, 2, 128, 128, 3, None) == INVALID  # length not a multiple of B
    assert g(A, A, A, A, A, cu(0, 512, 256), 2, 2, 128, 128, 3, None) == INVALID  # decreasing offsets
    assert g(A, A, A, A, A, cu(0, 0, 0), 2, 2, 128, 128, 3, None) == INVALID      # no tokens
    assert g(A, A, A, A, A, ok, 513, 2, 128, 128, 3, None) == UNSUPPORTED         # too many sequences
    assert g(A, A, A, A, A, cu(0, 128 * 40, 128 * 41), 2, 2, 128, 128, 33, None) == UNSUPPORTED
    assert g(None, A, A, A, A, ok, 2, 2, 128, 128, 3, None) == INVALID
    assert lib.moba_gate_topk_varlen(A, A, A, cu(0, 300), 1, 2, 128, 128, 3, None) == INVALID
    assert lib.moba_prefill_bwd_varlen(A, A, A, A, A, A, A, A, A, ok, 2, 2, 96, 128, 3, None) == UNSUPPORTED


def test_no_device_is_a_hip_error(lib):
    """Without a GPU, calls whose arguments pass the checks stop at the device
    lookup with MOBA_ERR_HIP and the HIP error kept for moba_last_hip_error
    (on a machine with a GPU these fake pointers must never reach a kernel, so
    the test only runs where there is none)."""
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present: the fake pointers would be launched on")
    HIP_ERROR_NO_DEVICE = 100
    calls = [
        lambda: prefill(lib),
        lambda: prefill(lib, f32=True),
        lambda: gate(lib),
        lambda: pool(lib),
        lambda: decode(lib),
        lambda: backward(lib),
        lambda: lib.moba_block_query_lists(A, A, A, A, A, 3328, 1024, 2, 128, 128, 3, None),
        lambda: lib.moba_decode_fwd_noalloc(A, A, A, None, 0, A, A, None, 1000, 2, 128, 128, 3, None),
    ]
    for i, call in enumerate(calls):
        assert call() == 3, i
        assert lib.moba_last_hip_error() == HIP_ERROR_NO_DEVICE, i
