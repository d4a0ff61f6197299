"""Python binding of libmoba, the MI355X (gfx950) MoBA causal prefill library.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C-ABI declared in ``include/moba.h``. PyTorch provides the
device memory and the current stream. There is no fallback: if ``libmoba.so``
is missing or a call fails, an exception is raised.

Tensors are row-major ``[N, H, D]`` (token, head, dim) on a CUDA (HIP) device,
bf16 or fp32; ``lse`` is ``[H, N]`` fp32; ``sel`` is ``[H, N, topk]`` int32.
"""

from __future__ import annotations

import ctypes
import os

__all__ = ["prefill", "gate_topk", "block_mean_keys", "block_query_lists", "MobaError", "library_path", "load_library",
           "StageEvents", "STAGES", "STATUS", "MAX_TOPK", "MAX_BLOCKS", "debug_poison_workspace"]

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOBA_LIBRARY selects another build of the library (the host-sanitized debug
# build); by default the in-tree libmoba.so is loaded.
_LIB_PATH = os.environ.get("MOBA_LIBRARY") or os.path.join(_HERE, "libmoba.so")
_lib = None

STATUS = {0: "MOBA_OK", 1: "MOBA_ERR_INVALID_ARG", 2: "MOBA_ERR_UNSUPPORTED", 3: "MOBA_ERR_HIP",
          4: "MOBA_ERR_OUT_OF_MEMORY"}
MAX_TOPK = 32
MAX_BLOCKS = 4096

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32

_SIGNATURES = {
    "moba_block_mean_keys": [_P, _P, _I64, _I32, _I32, _I32, _P],
    "moba_block_mean_keys_f32": [_P, _P, _I64, _I32, _I32, _I32, _P],
    "moba_gate_topk": [_P, _P, _P, _I64, _I32, _I32, _I32, _I32, _P],
    "moba_gate_topk_f32": [_P, _P, _P, _I64, _I32, _I32, _I32, _I32, _P],
    "moba_block_query_lists": [_P, _P, _P, _P, _P, _I64, _I64, _I32, _I32, _I32, _I32, _P],
    "moba_prefill_fwd": [_P, _P, _P, _P, _P, _I64, _I32, _I32, _I32, _I32, _P],
    "moba_prefill_fwd_f32": [_P, _P, _P, _P, _P, _I64, _I32, _I32, _I32, _I32, _P],
    "moba_prefill_fwd_timed": [_P, _P, _P, _P, _P, _I64, _I32, _I32, _I32, _I32, _P, _P],
    "moba_decode_fwd": [_P, _P, _P, _P, _I32, _P, _P, _P, _I64, _I32, _I32, _I32, _I32, _P],
    "moba_prefill_bwd": [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I64, _I32, _I32, _I32, _I32, _P],
    "moba_block_pool_keys": [_P, _P, _P, _I64, _I32, _I32, _I32, _I32, _P],
    "moba_gate_topk_pooled": [_P, _P, _P, _P, _I64, _I32, _I32, _I32, _I32, _I32, _P],
    "moba_prefill_fwd_pooled": [_P, _P, _P, _P, _P, _P, _I64, _I32, _I32, _I32, _I32, _I32, _P],
    "moba_prefill_bwd_pooled": [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I64, _I32, _I32, _I32, _I32, _I32, _P],
    "moba_topk_for_sparsity": [_I64, _I32, ctypes.c_double],
    "moba_gate_topk_varlen": [_P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _P],
    "moba_prefill_fwd_varlen": [_P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _P],
    "moba_prefill_bwd_varlen": [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _P],
    "moba_decode_fwd_noalloc": [_P, _P, _P, _P, _I32, _P, _P, _P, _I64, _I32, _I32, _I32, _I32, _P],
    "moba_debug_poison_workspace": [ctypes.c_int],
    "moba_status_string": [ctypes.c_int],
    "moba_last_hip_error": [],
}


class MobaError(RuntimeError):
    def __init__(self, status: int, where: str, hip_error: int = 0):
        name = STATUS.get(status, f"status {status}")
        msg = f"{where}: {name}" + (f" (hipError {hip_error})" if status == 3 else "")
        super().__init__(msg)
        self.status = status
        self.hip_error = hip_error


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libmoba.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        # torch ships its own HIP runtime; importing it first makes the library
        # bind to that one instead of loading a second runtime into the process.
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`")
        lib = ctypes.CDLL(_LIB_PATH)
        for name, args in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = ctypes.c_char_p if name == "moba_status_string" else ctypes.c_int
        lib.moba_topk_for_sparsity.restype = ctypes.c_int32
        _lib = lib
    return _lib


def debug_poison_workspace(on: bool) -> bool:
    """Switch the library's workspace poisoning on or off (every later call
    fills its workspace with 0xFF bytes before its first stage); returns the
    previous setting."""
    return bool(load_library().moba_debug_poison_workspace(1 if on else 0))


def _check(status: int, where: str):
    if status != 0:
        raise MobaError(status, where, load_library().moba_last_hip_error() if status == 3 else 0)


def _stream(device):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check_qkv(*ts):
    import torch
    t0 = ts[0]
    if t0.dim() != 3:
        raise ValueError("expected [N, H, D] tensors")
    if t0.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("tensors must be bfloat16 or float32")
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must be on a GPU device")
        if t.shape != t0.shape or t.dtype != t0.dtype or t.device != t0.device:
            raise ValueError("q, k, v must share shape, dtype and device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous [N, H, D]")
    N, H, D = t0.shape
    return N, H, D, t0.dtype == torch.float32


def block_mean_keys(k, block_size: int):
    """Block mean keys, fp32 ``[H, N // block_size, D]``."""
    import torch
    N, H, D, f32 = _check_qkv(k)
    lib = load_library()
    n = N // block_size if block_size > 0 else 0
    kbar = torch.empty((H, max(n, 1), D), dtype=torch.float32, device=k.device)
    fn = lib.moba_block_mean_keys_f32 if f32 else lib.moba_block_mean_keys
    _check(fn(k.data_ptr(), kbar.data_ptr(), N, H, D, block_size, _stream(k.device)), "moba_block_mean_keys")
    return kbar


def gate_topk(q, k, block_size: int, topk: int):
    """Chosen blocks per (head, query): int32 ``[H, N, topk]``, ascending, -1 padded."""
    import torch
    N, H, D, f32 = _check_qkv(q, k)
    lib = load_library()
    sel = torch.empty((H, N, max(topk, 1)), dtype=torch.int32, device=q.device)
    fn = lib.moba_gate_topk_f32 if f32 else lib.moba_gate_topk
    _check(fn(q.data_ptr(), k.data_ptr(), sel.data_ptr(), N, H, D, block_size, topk, _stream(q.device)),
           "moba_gate_topk")
    return sel


def block_query_lists(q, k, block_size: int, topk: int):
    """The prefill's selection and its per-block query lists.

    Returns ``(sel, offs, qidx)``: ``sel`` int32 ``[H, N, topk]`` as
    ``gate_topk``; list ``(h, b)`` is ``qidx[offs[h*n + b]:offs[h*n + b + 1]]``,
    the ascending positions of the queries that chose ``b`` as a past block.
    """
    import torch
    N, H, D, f32 = _check_qkv(q, k)
    if f32:
        raise TypeError("block_query_lists takes bfloat16 q and k")
    lib = load_library()
    n = N // block_size if block_size > 0 and N % block_size == 0 else 0
    # Buffer size: every query of block j keeps min(topk - 1, j) past blocks.
    pairs = H * sum(block_size * min(topk - 1, j) for j in range(n)) if topk >= 1 else 0
    sel = torch.empty((H, N, max(topk, 1)), dtype=torch.int32, device=q.device)
    offs = torch.empty((H * n + 1,), dtype=torch.int32, device=q.device)
    qidx = torch.empty((max(pairs, 1),), dtype=torch.int32, device=q.device)
    _check(lib.moba_block_query_lists(q.data_ptr(), k.data_ptr(), sel.data_ptr(), offs.data_ptr(), qidx.data_ptr(),
                                      pairs, N, H, D, block_size, topk, _stream(q.device)),
           "moba_block_query_lists")
    return sel, offs, qidx[:pairs]


STAGES = ("pool", "gate", "lists", "attn_past", "attn_own", "merge")
STAGE_EVENTS = len(STAGES) + 1


class StageEvents:
    """HIP events the library records at its stage boundaries (bf16 prefill).

    ``stages`` limits the recorded boundaries to those around the named stages
    (the others are passed as NULL and not recorded); their times accumulate
    in ``totals``, the other stages stay at zero."""

    def __init__(self, stages=STAGES):
        self._hip = ctypes.CDLL("libamdhip64.so")
        self._hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self._hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self._hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self._hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.stages = tuple(stages)
        wanted = set()
        for s in self.stages:
            i = STAGES.index(s)
            wanted.update((i, i + 1))
        self.array = (ctypes.c_void_p * STAGE_EVENTS)()
        for i in range(STAGE_EVENTS):
            self.array[i] = None
            if i in wanted:
                ev = ctypes.c_void_p()
                if self._hip.hipEventCreate(ctypes.byref(ev)) != 0:
                    raise RuntimeError("hipEventCreate failed")
                self.array[i] = ev
        self.totals = {s: 0.0 for s in STAGES}
        self.calls = 0

    def accumulate(self):
        """Wait for the last recorded call and add its stage times (ms)."""
        last = max(i for i in range(STAGE_EVENTS) if self.array[i])
        if self._hip.hipEventSynchronize(self.array[last]) != 0:
            raise RuntimeError("hipEventSynchronize failed")
        ms = ctypes.c_float()
        for s in self.stages:
            i = STAGES.index(s)
            if self._hip.hipEventElapsedTime(ctypes.byref(ms), self.array[i], self.array[i + 1]) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            self.totals[s] += ms.value
        self.calls += 1

    def mean_ms(self):
        return {s: v / max(self.calls, 1) for s, v in self.totals.items()}

    def close(self):
        for i in range(STAGE_EVENTS):
            if self.array[i]:
                self._hip.hipEventDestroy(self.array[i])


def prefill(q, k, v, block_size: int, topk: int, out=None, lse=None, events: "StageEvents | None" = None):
    """MoBA causal prefill. Returns ``(out [N,H,D], lse [H,N] fp32)``.

    ``events`` (bf16 only) records the stage boundaries for timing."""
    import torch
    N, H, D, f32 = _check_qkv(q, k, v)
    lib = load_library()
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((H, N), dtype=torch.float32, device=q.device)
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor like q")
    if lse.shape != (H, N) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous fp32 [H, N] tensor")
    if events is not None:
        if f32:
            raise ValueError("stage events are recorded by the bf16 prefill only")
        _check(lib.moba_prefill_fwd_timed(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                          N, H, D, block_size, topk, _stream(q.device), events.array),
               "moba_prefill_fwd_timed")
        return out, lse
    fn = lib.moba_prefill_fwd_f32 if f32 else lib.moba_prefill_fwd
    _check(fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), N, H, D, block_size, topk,
              _stream(q.device)), "moba_prefill_fwd")
    return out, lse


POOLING = {"mean": 0, "max": 1, "weighted": 2}


def _pool_args(pooling, weights, H, N, device):
    import torch
    if pooling not in POOLING:
        raise ValueError(f"pooling must be one of {sorted(POOLING)}")
    if pooling == "weighted":
        if weights is None or weights.shape != (H, N) or weights.dtype != torch.float32 \
                or not weights.is_contiguous() or weights.device != device:
            raise ValueError("weighted pooling needs contiguous fp32 [H, N] weights on the inputs' device")
        return POOLING[pooling], weights.data_ptr()
    return POOLING[pooling], None


def block_pool_keys(k, block_size: int, pooling: str = "mean", weights=None):
    """Pooled block keys (bf16 k), fp32 ``[H, N // block_size, D]``; ``pooling`` is
    "mean", "max" or "weighted" (``weights`` fp32 [H, N], non-negative)."""
    import torch
    N, H, D, f32 = _check_qkv(k)
    if f32:
        raise TypeError("block_pool_keys takes bf16 keys")
    mode, wp = _pool_args(pooling, weights, H, N, k.device)
    lib = load_library()
    kbar = torch.empty((H, max(N // block_size, 1), D), dtype=torch.float32, device=k.device)
    _check(lib.moba_block_pool_keys(k.data_ptr(), wp, kbar.data_ptr(), N, H, D, block_size, mode, _stream(k.device)),
           "moba_block_pool_keys")
    return kbar


def gate_topk_pooled(q, k, block_size: int, topk: int, pooling: str = "mean", weights=None):
    """:func:`gate_topk` (bf16) with the block keys pooled by ``pooling``."""
    import torch
    N, H, D, f32 = _check_qkv(q, k)
    if f32:
        raise TypeError("the pooled gate takes bf16 tensors")
    mode, wp = _pool_args(pooling, weights, H, N, q.device)
    lib = load_library()
    sel = torch.empty((H, N, max(topk, 1)), dtype=torch.int32, device=q.device)
    _check(lib.moba_gate_topk_pooled(q.data_ptr(), k.data_ptr(), wp, sel.data_ptr(), N, H, D, block_size, topk, mode,
                                     _stream(q.device)), "moba_gate_topk_pooled")
    return sel


def prefill_pooled(q, k, v, block_size: int, topk: int, pooling: str = "mean", weights=None, out=None, lse=None):
    """:func:`prefill` (bf16) with the gate's block keys pooled by ``pooling``."""
    import torch
    N, H, D, f32 = _check_qkv(q, k, v)
    if f32:
        raise TypeError("the pooled prefill takes bf16 tensors")
    mode, wp = _pool_args(pooling, weights, H, N, q.device)
    lib = load_library()
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor like q")
    if lse.shape != (H, N) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous fp32 [H, N] tensor")
    _check(lib.moba_prefill_fwd_pooled(q.data_ptr(), k.data_ptr(), v.data_ptr(), wp, out.data_ptr(), lse.data_ptr(),
                                       N, H, D, block_size, topk, mode, _stream(q.device)), "moba_prefill_fwd_pooled")
    return out, lse


def _cu(cu_seqlens):
    """Host int64 copy of cu_seqlens (a list, numpy array or CPU tensor) and its ctypes pointer."""
    import numpy as np
    arr = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    if arr.ndim != 1 or arr.size < 2:
        raise ValueError("cu_seqlens must hold num_seqs + 1 offsets")
    return arr, arr.ctypes.data_as(ctypes.c_void_p), arr.size - 1


def gate_topk_varlen(q, k, cu_seqlens, block_size: int, topk: int):
    """Selections of packed sequences (bf16): int32 ``[H, T, topk]``, global block indices."""
    import torch
    T, H, D, f32 = _check_qkv(q, k)
    if f32:
        raise TypeError("packed sequences take bf16 tensors")
    arr, cp, S = _cu(cu_seqlens)
    lib = load_library()
    sel = torch.empty((H, T, max(topk, 1)), dtype=torch.int32, device=q.device)
    _check(lib.moba_gate_topk_varlen(q.data_ptr(), k.data_ptr(), sel.data_ptr(), cp, S, H, D, block_size, topk,
                                     _stream(q.device)), "moba_gate_topk_varlen")
    return sel


def prefill_varlen(q, k, v, cu_seqlens, block_size: int, topk: int, out=None, lse=None):
    """MoBA prefill of packed sequences (bf16 ``[T, H, D]``): ``(out, lse [H, T])``."""
    import torch
    T, H, D, f32 = _check_qkv(q, k, v)
    if f32:
        raise TypeError("packed sequences take bf16 tensors")
    arr, cp, S = _cu(cu_seqlens)
    lib = load_library()
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((H, T), dtype=torch.float32, device=q.device) if lse is None else lse
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor like q")
    if lse.shape != (H, T) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous fp32 [H, T] tensor")
    _check(lib.moba_prefill_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), cp,
                                       S, H, D, block_size, topk, _stream(q.device)), "moba_prefill_fwd_varlen")
    return out, lse


def prefill_backward_varlen(q, k, v, out, lse, dout, cu_seqlens, block_size: int, topk: int):
    """Gradients of :func:`prefill_varlen`: ``(dq, dk, dv)`` bf16 ``[T, H, D]``."""
    import torch
    T, H, D, f32 = _check_qkv(q, k, v, out, dout)
    if f32:
        raise TypeError("packed sequences take bf16 tensors")
    if lse.shape != (H, T) or lse.dtype != torch.float32 or not lse.is_contiguous() or lse.device != q.device:
        raise ValueError("lse must be a contiguous fp32 [H, T] tensor on q's device")
    arr, cp, S = _cu(cu_seqlens)
    lib = load_library()
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    _check(lib.moba_prefill_bwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                       dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), cp, S, H, D,
                                       block_size, topk, _stream(q.device)), "moba_prefill_bwd_varlen")
    return dq, dk, dv


def topk_for_sparsity(N: int, block_size: int, sparsity: float) -> int:
    """Dynamic k: the top_k keeping a late query's sparsity at ``sparsity`` (host only)."""
    k = load_library().moba_topk_for_sparsity(N, block_size, sparsity)
    if k < 1:
        raise MobaError(-k, "moba_topk_for_sparsity")
    return k


def prefill_backward(q, k, v, out, lse, dout, block_size: int, topk: int, dq=None, dk=None, dv=None,
                     pooling: str = "mean", weights=None):
    """Gradients of the bf16 MoBA prefill output: returns ``(dq, dk, dv)`` [N, H, D] bf16.

    ``out`` and ``lse`` are what :func:`prefill` returned for the same inputs;
    ``dout`` is the upstream gradient of ``out``. The top-k selection carries
    no gradient (it is recomputed and held fixed)."""
    import torch
    N, H, D, f32 = _check_qkv(q, k, v, out, dout)
    if f32:
        raise TypeError("the backward pass takes bf16 tensors")
    if lse.shape != (H, N) or lse.dtype != torch.float32 or not lse.is_contiguous() or lse.device != q.device:
        raise ValueError("lse must be a contiguous fp32 [H, N] tensor on q's device")
    grads = []
    for g in (dq, dk, dv):
        if g is None:
            g = torch.empty_like(q)
        elif g.shape != q.shape or g.dtype != q.dtype or not g.is_contiguous() or g.device != q.device:
            raise ValueError("dq, dk, dv must be contiguous tensors like q")
        grads.append(g)
    lib = load_library()
    if pooling == "mean":
        _check(lib.moba_prefill_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                    dout.data_ptr(), grads[0].data_ptr(), grads[1].data_ptr(), grads[2].data_ptr(),
                                    N, H, D, block_size, topk, _stream(q.device)), "moba_prefill_bwd")
    else:
        mode, wp = _pool_args(pooling, weights, H, N, q.device)
        _check(lib.moba_prefill_bwd_pooled(q.data_ptr(), k.data_ptr(), v.data_ptr(), wp, out.data_ptr(),
                                           lse.data_ptr(), dout.data_ptr(), grads[0].data_ptr(), grads[1].data_ptr(),
                                           grads[2].data_ptr(), N, H, D, block_size, topk, mode, _stream(q.device)),
               "moba_prefill_bwd_pooled")
    return tuple(grads)


def decode(q_new, k, v, block_size: int, topk: int, kbar=None, out=None, lse=None, sel=None, noalloc=False):
    """MoBA decode step (bf16) for the token at position N - 1 of the cache.

    ``q_new`` [H, D]; ``k``, ``v`` [N, H, D] (the token's own key and value are
    the last rows); ``kbar`` optional fp32 [H, nb, D] block means of the
    complete blocks (nb >= (N - 1) // block_size), e.g. from
    :func:`block_mean_keys` over the complete prefix. Returns
    ``(out [H, D] bf16, lse [H] fp32)``; ``sel`` (int32 [H, topk]) receives
    the kept blocks when given. ``noalloc`` calls the allocation-free entry
    point (workspace in the library's fixed per-GPU scratch array)."""
    import torch
    if k.dim() != 3 or k.dtype != torch.bfloat16 or not k.is_cuda:
        raise ValueError("k must be a bf16 [N, H, D] GPU tensor")
    N, H, D = k.shape
    for t in (k, v):
        if t.shape != k.shape or t.dtype != k.dtype or t.device != k.device or not t.is_contiguous():
            raise ValueError("k and v must be contiguous bf16 [N, H, D] tensors on one device")
    if q_new.shape != (H, D) or q_new.dtype != torch.bfloat16 or q_new.device != k.device or not q_new.is_contiguous():
        raise ValueError("q_new must be a contiguous bf16 [H, D] tensor on the cache's device")
    lib = load_library()
    if out is None:
        out = torch.empty_like(q_new)
    if lse is None:
        lse = torch.empty((H,), dtype=torch.float32, device=k.device)
    kb, nb = 0, 0
    if kbar is not None:
        if kbar.dim() != 3 or kbar.shape[0] != H or kbar.shape[2] != D or kbar.dtype != torch.float32 \
                or not kbar.is_contiguous():
            raise ValueError("kbar must be a contiguous fp32 [H, nb, D] tensor")
        kb, nb = kbar.data_ptr(), kbar.shape[1]
    sp = 0
    if sel is not None:
        if sel.shape != (H, topk) or sel.dtype != torch.int32 or not sel.is_contiguous():
            raise ValueError("sel must be a contiguous int32 [H, topk] tensor")
        sp = sel.data_ptr()
    fn, name = (lib.moba_decode_fwd_noalloc, "moba_decode_fwd_noalloc") if noalloc else \
        (lib.moba_decode_fwd, "moba_decode_fwd")
    _check(fn(q_new.data_ptr(), k.data_ptr(), v.data_ptr(), kb, nb, out.data_ptr(), lse.data_ptr(),
              sp, N, H, D, block_size, topk, _stream(k.device)), name)
    return out, lse
