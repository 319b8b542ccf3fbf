"""Seeded synthetic inputs for the Infini-attention forward pass.

This module only *draws and stores* numbers: it holds none of the method's
arithmetic. Both the fp64 oracle and the GPU path consume exactly the arrays it
returns, so a parity comparison always starts from identical, already-rounded
inputs.

Recipe (one definition, used everywhere):

* Generator: ``numpy.random.default_rng(seed)`` (PCG64).
* Draw order: Q, K, V, each ``standard_normal(shape) / sqrt(d)`` in fp64 over the
  flattened ``[B, H, L, d]`` order, then beta (one value per query head), then,
  for configurations with outlier keys, the outlier positions per (b, kv-head)
  in (b, h) order, drawn without replacement; those K rows are scaled by the
  outlier factor *before* rounding.
* Rounding: fp64 -> fp32 (round to nearest even), and for bf16 storage
  fp32 -> bf16 (round to nearest even on the bit pattern). bf16 tensors are
  handed around as ``uint16`` bit patterns.
* Initial state: ``M0 = 0``, ``z0 = 0`` (fp32), eps = 1e-6.

The five workload shapes are the model and context scales the pages quote
(segment length 64 with rollout 16 for a 200M model; a 300M LLaMA at 16,384
tokens; the Llama-3-8B attention shape; contexts beyond one million tokens).
Gaussian inputs stand in for the language-modelling, passkey and summarisation
data those pages evaluate on, which are not used here.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional, Tuple

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "round_fp32",
    "round_bf16_bits",
    "bf16_bits_to_f32",
    "as_f64",
    "generate",
    "random_case",
    "random_cotangents",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    d: int
    seg_len: int
    seq_len: int
    dtype: str  # "f32" or "bf16": storage type of q, k, v and out
    modes: Tuple[str, ...]  # update rules exercised: "linear", "delta"
    beta_dist: str  # "normal:<var>" or "uniform:<lo>:<hi>"
    seed: int
    outlier_frac: float = 0.0
    outlier_scale: float = 1.0
    eps: float = 1e-6

    @property
    def n_segments(self) -> int:
        return -(-self.seq_len // self.seg_len)

    @property
    def tokens(self) -> int:
        return self.batch * self.seq_len

    def describe(self) -> str:
        return (
            f"{self.name}: B={self.batch} Hq={self.n_q_heads} Hkv={self.n_kv_heads} "
            f"d={self.d} N={self.seg_len} L={self.seq_len} S={self.n_segments} {self.dtype}"
        )


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("tiny_f32", 1, 2, 2, 32, 64, 256, "f32", ("linear",), "normal:1", seed=1),
        Workload("small_200m", 2, 8, 8, 64, 64, 1024, "bf16", ("linear", "delta"),
                 "uniform:-4:4", seed=2),
        Workload("llama300m_16k", 4, 16, 16, 64, 2048, 16384, "bf16", ("delta",), "normal:2",
                 seed=3, outlier_frac=0.05, outlier_scale=4.0),
        Workload("llama3_8b_gqa", 1, 32, 8, 128, 2048, 32768, "bf16", ("linear", "delta"),
                 "normal:1", seed=4),
        Workload("stream_1m", 1, 8, 8, 128, 2048, 1048576, "bf16", ("delta",), "normal:1",
                 seed=5),
    ]
}


# ----------------------------------------------------------------------------
# storage formats
# ----------------------------------------------------------------------------

def round_fp32(x: np.ndarray) -> np.ndarray:
    """fp64 -> fp32 with IEEE round-to-nearest-even (numpy's cast)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def round_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even.

    NaN keeps a quiet-NaN pattern; infinities and overflow behave as IEEE RNE.
    """
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    r = np.where(nan, (u >> np.uint32(16)) | np.uint32(0x0040), r)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def as_f64(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Exact upcast of a stored tensor ("f32" array or "bf16" bits) to fp64."""
    if dtype == "bf16":
        return bf16_bits_to_f32(arr).astype(np.float64)
    return np.asarray(arr, dtype=np.float32).astype(np.float64)


def _store(x64: np.ndarray, dtype: str) -> np.ndarray:
    x32 = round_fp32(x64)
    if dtype == "bf16":
        return round_bf16_bits(x32)
    return x32


def _draw_beta(rng: np.random.Generator, n: int, dist: str) -> np.ndarray:
    kind, *par = dist.split(":")
    if kind == "normal":
        var = float(par[0])
        return round_fp32(rng.standard_normal(n) * math.sqrt(var))
    if kind == "uniform":
        lo, hi = float(par[0]), float(par[1])
        return round_fp32(rng.uniform(lo, hi, n))
    raise ValueError(f"unknown beta distribution {dist!r}")


def _draw_qkv(rng: np.random.Generator, shape: Tuple[int, ...], d: int, dtype: str,
              chunk: int = 1 << 24) -> np.ndarray:
    """Draw standard_normal(shape)/sqrt(d) in flattened order, in chunks, and store."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16 if dtype == "bf16" else np.float32)
    inv = 1.0 / math.sqrt(d)
    pos = 0
    while pos < n:
        m = min(chunk, n - pos)
        out[pos:pos + m] = _store(rng.standard_normal(m) * inv, dtype)
        pos += m
    return out.reshape(shape)


def generate(w: Workload, seq_len: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Seeded inputs for workload ``w`` (optionally truncated to ``seq_len`` tokens).

    Truncation draws the same recipe at the shorter length (it is a smaller
    workload with the same seed, not a prefix of the full one).
    Returns q, k, v (storage dtype), beta, M0, z0 (fp32) and eps.
    """
    L = w.seq_len if seq_len is None else seq_len
    rng = np.random.default_rng(w.seed)
    B, Hq, Hkv, d = w.batch, w.n_q_heads, w.n_kv_heads, w.d
    q = _draw_qkv(rng, (B, Hq, L, d), d, w.dtype)
    if w.outlier_frac > 0.0:
        # K needs the outlier rows scaled before rounding: draw in fp64 per (b, h).
        k64 = rng.standard_normal((B, Hkv, L, d)) / math.sqrt(d)
    else:
        k = _draw_qkv(rng, (B, Hkv, L, d), d, w.dtype)
    v = _draw_qkv(rng, (B, Hkv, L, d), d, w.dtype)
    beta = _draw_beta(rng, Hq, w.beta_dist)
    if w.outlier_frac > 0.0:
        n_out = int(math.floor(w.outlier_frac * L))
        for b in range(B):
            for h in range(Hkv):
                rows = rng.choice(L, size=n_out, replace=False)
                k64[b, h, rows, :] *= w.outlier_scale
        k = _store(k64, w.dtype)
        del k64
    M0 = np.zeros((B, Hkv, d, d), dtype=np.float32)
    z0 = np.zeros((B, Hkv, d), dtype=np.float32)
    return dict(q=q, k=k, v=v, beta=beta, M0=M0, z0=z0, eps=np.float32(w.eps))


def random_case(seed: int, B: int, Hq: int, Hkv: int, L: int, dk: int, dv: int,
                dtype: str = "f32", scale: Optional[float] = None,
                beta: Optional[np.ndarray] = None, nonzero_state: bool = False,
                positive: bool = False) -> Dict[str, np.ndarray]:
    """Small seeded case with arbitrary (distinct) axis sizes for tests.

    ``scale`` multiplies the N(0,1) draws (default 1/sqrt(dk)); ``positive`` takes
    absolute values (all entries > 0); ``nonzero_state`` draws a nonnegative M0,
    z0 instead of zeros.
    """
    rng = np.random.default_rng(seed)
    s = (1.0 / math.sqrt(dk)) if scale is None else scale

    def draw(shape):
        x = rng.standard_normal(shape) * s
        if positive:
            x = np.abs(x)
        return _store(x, dtype)

    q = draw((B, Hq, L, dk))
    k = draw((B, Hkv, L, dk))
    v = draw((B, Hkv, L, dv))
    b = round_fp32(rng.standard_normal(Hq)) if beta is None else round_fp32(np.asarray(beta))
    if nonzero_state:
        M0 = round_fp32(rng.standard_normal((B, Hkv, dk, dv)))
        z0 = round_fp32(np.abs(rng.standard_normal((B, Hkv, dk))) * 4.0 + 1.0)
    else:
        M0 = np.zeros((B, Hkv, dk, dv), dtype=np.float32)
        z0 = np.zeros((B, Hkv, dk), dtype=np.float32)
    return dict(q=q, k=k, v=v, beta=b, M0=M0, z0=z0, eps=np.float32(1e-6))



def random_cotangents(seed: int, B: int, Hq: int, Hkv: int, L: int, d: int, dtype: str = "f32",
                      state: bool = True) -> Dict[str, Optional[np.ndarray]]:
    """Seeded gradients of a loss with respect to the forward's outputs: d_out
    [B, Hq, L, d] in the storage dtype, and (when ``state``) d_M [B, Hkv, d, d],
    d_z [B, Hkv, d] in fp32; N(0, 1) draws in that order."""
    rng = np.random.default_rng(seed)
    d_out = _store(rng.standard_normal((B, Hq, L, d)), dtype)
    if not state:
        return dict(d_out=d_out, d_M=None, d_z=None)
    d_M = round_fp32(rng.standard_normal((B, Hkv, d, d)))
    d_z = round_fp32(rng.standard_normal((B, Hkv, d)))
    return dict(d_out=d_out, d_M=d_M, d_z=d_z)
