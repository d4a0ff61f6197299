"""Seeded synthetic inputs for MoBA causal prefill.

This module only draws random tensors with the shapes and value structure of the
workloads; it holds none of the method's arithmetic (no pooling, gating,
selection or attention). Both the fp64 oracle tests and the HIP path take their
inputs from here, so the two sides see identical bits.

Layout of every generated tensor: ``[N, H, D]`` row-major (token, head, dim),
float32 numpy arrays. For bf16 workloads the float32 values are already rounded
to bf16 (round to nearest even), so widening them to fp64 on the oracle side and
narrowing them to ``torch.bfloat16`` on the device side are both exact.

Workloads (one sequence, batch 1, H query heads = H key/value heads):

==== ========= === === ====== ==== ===== ===========================================
name N         H   D   block  n    top_k values
==== ========= === === ====== ==== ===== ===========================================
tiny 2048      1   64  256    8    3     fp32 N(0,1)
c32k 32768     1   128 2048   16   3     bf16 N(0,1); per-block key offset
                                         N(0, 0.5^2) shared by the block's keys
h32  32768     32  128 512    64   3     bf16 N(0,1)/sqrt(128); per-head seeds
n128k 131072   8   128 4096   32   12    bf16 N(0,1) + 4 planted needle blocks
m1   1048576   1   128 4096   256  12    bf16 N(0,1); 4096 sampled rows
==== ========= === === ====== ==== ===== ===========================================
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    N: int
    H: int
    D: int
    block_size: int
    topk: int
    dtype: str          # "fp32" or "bf16"
    description: str

    @property
    def n_blocks(self) -> int:
        return self.N // self.block_size


WORKLOADS = {
    "tiny": Workload("tiny", 2048, 1, 64, 256, 3, "fp32",
                     "N=2048 H=1 D=64 B=256 top-3, fp32 N(0,1), seed 0"),
    "c32k": Workload("c32k", 32768, 1, 128, 2048, 3, "bf16",
                     "N=32768 H=1 D=128 B=2048 top-3, bf16 N(0,1), per-block key offset N(0,0.5^2), seed 1"),
    "h32": Workload("h32", 32768, 32, 128, 512, 3, "bf16",
                    "N=32768 H=32 D=128 B=512 top-3, bf16 N(0,1)/sqrt(128), per-head seeds [2,h]"),
    "n128k": Workload("n128k", 131072, 8, 128, 4096, 12, "bf16",
                      "N=131072 H=8 D=128 B=4096 top-12, bf16 N(0,1) + 4 needle blocks/head, seeds [3,h]"),
    "m1": Workload("m1", 1048576, 1, 128, 4096, 12, "bf16",
                   "N=1048576 H=1 D=128 B=4096 top-12, bf16 N(0,1), seed 4"),
}

# Strength of the planted needle direction added to every key of a needle block.
NEEDLE_STRENGTH = 0.5
NEEDLE_BLOCKS = 4
# Standard deviation of the per-block key offset of the "c32k" workload.
BLOCK_OFFSET_STD = 0.5


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    bias = ((bits >> 16) & 1) + 0x7FFF
    out = ((bits + bias) & 0xFFFF0000).astype(np.uint32)
    return out.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bf16-representable (int16 view)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16).view(np.int16)


def _normal(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(shape, dtype=np.float32)


def make_qkv(N: int, H: int, D: int, seed, dtype: str = "bf16", scale: float = 1.0):
    """Plain i.i.d. N(0, scale^2) q, k, v of shape [N, H, D], drawn in that order."""
    rng = np.random.default_rng(seed)
    q = _normal(rng, (N, H, D))
    k = _normal(rng, (N, H, D))
    v = _normal(rng, (N, H, D))
    if scale != 1.0:
        q *= np.float32(scale)
        k *= np.float32(scale)
        v *= np.float32(scale)
    if dtype == "bf16":
        q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
    return q, k, v


def make_grad(N: int, H: int, D: int, seed, dtype: str = "bf16", scale: float = 1.0):
    """An upstream gradient dO for the backward pass: i.i.d. N(0, scale^2), [N, H, D]."""
    rng = np.random.default_rng(seed)
    g = _normal(rng, (N, H, D))
    if scale != 1.0:
        g *= np.float32(scale)
    return round_to_bf16(g) if dtype == "bf16" else g


def _per_head(N, H, D, seed_of_head, fill):
    q = np.empty((N, H, D), np.float32)
    k = np.empty((N, H, D), np.float32)
    v = np.empty((N, H, D), np.float32)
    extras = []
    for h in range(H):
        rng = np.random.default_rng(seed_of_head(h))
        qh, kh, vh, ex = fill(rng)
        q[:, h, :], k[:, h, :], v[:, h, :] = qh, kh, vh
        extras.append(ex)
    return q, k, v, extras


def make_workload(name: str, with_extras: bool = False):
    """Inputs of a named workload: returns (Workload, q, k, v) as float32 [N,H,D].

    With ``with_extras`` a fifth item is returned: a dict that, for "n128k",
    holds the planted needle blocks of every head under "needle_blocks".
    """
    w = WORKLOADS[name]
    N, H, D, B = w.N, w.H, w.D, w.block_size
    n = w.n_blocks
    extras = {}
    if name == "tiny":
        q, k, v = make_qkv(N, H, D, 0, dtype="fp32")
    elif name == "c32k":
        rng = np.random.default_rng(1)
        q = _normal(rng, (N, H, D))
        k = _normal(rng, (N, H, D))
        v = _normal(rng, (N, H, D))
        off = _normal(rng, (n, H, D)) * np.float32(BLOCK_OFFSET_STD)
        k = (k.reshape(n, B, H, D) + off[:, None, :, :]).reshape(N, H, D)
        q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
    elif name == "h32":
        s = np.float32(1.0 / math.sqrt(D))

        def fill(rng):
            return _normal(rng, (N, D)) * s, _normal(rng, (N, D)) * s, _normal(rng, (N, D)) * s, None
        q, k, v, _ = _per_head(N, H, D, lambda h: [2, h], fill)
        q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
    elif name == "n128k":
        def fill(rng):
            qh, kh, vh = _normal(rng, (N, D)), _normal(rng, (N, D)), _normal(rng, (N, D))
            r = int(rng.integers(0, N))
            u = qh[r] / np.linalg.norm(qh[r])
            blocks = rng.choice(n - 1, size=NEEDLE_BLOCKS, replace=False)
            for b in blocks:
                kh[b * B:(b + 1) * B] += np.float32(NEEDLE_STRENGTH) * u
            return qh, kh, vh, sorted(int(b) for b in blocks)
        q, k, v, needles = _per_head(N, H, D, lambda h: [3, h], fill)
        extras["needle_blocks"] = needles
        q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
    elif name == "m1":
        q, k, v = make_qkv(N, H, D, 4, dtype="bf16")
    else:  # pragma: no cover
        raise KeyError(name)
    if with_extras:
        return w, q, k, v, extras
    return w, q, k, v


def sample_rows(N: int, count: int, seed) -> np.ndarray:
    """Sorted distinct seeded query rows in [0, N)."""
    rng = np.random.default_rng(seed)
    count = min(count, N)
    return np.sort(rng.choice(N, size=count, replace=False)).astype(np.int64)


SAMPLE_SEED = {"n128k": 1003, "m1": 1004, "h32": 1002, "c32k": 1001, "tiny": 1000}
