"""Backward-pass throughput on one GPU.

    python -m compressive_memory_transformers_segment_amd.backward_bench [--steps K]

One step is one infini_attn_backward call over inputs already resident in HBM:
the gradients of <d_out, out> + <d_M, M_S> + <d_z, z_S> with respect to q, k,
v, beta and (M_0, z_0), taken through every segment in reverse. Shapes: the
Llama-3-8B attention shape (B = 1, 32 query heads over 8 kv heads, d = 128,
16 segments of 2048 rows, L = 32768) under both update rules, and the 300M
LLaMA-like layer (B = 4, 16 heads, d = 64, 8 segments of 2048, L = 16384),
delta rule, and the streaming long-context shape (B = 1, 8 heads, d = 128,
512 segments of 2048, L = 1048576), delta rule; bf16 storage. Inputs are seeded N(0, 1)/sqrt(d) values generated
on the device, d_out ~ N(0, 1), d_M = d_z = 0, M_0 = 0 and z_0 = 2048 (the
scale one earlier 2048-row segment leaves).

Each case prints one JSON line: milliseconds per call (HIP events on the launch
stream around K calls), tokens/s (B L per call), and algorithmic TFLOP/s. The
algorithmic count, per (query head, segment) of N rows and per (kv head,
segment):
  local attention backward  5 N^2 d  (QK^T recomputed, dO V^T, P^T dO, dS K,
                                      dS^T Q, each over the causal half)
  retrieval backward        6 N d^2  (sigma(Q) M recomputed, dnum M^T,
                                      sigma(Q)^T dnum)
  state recomputation       2 N d^2 linear, 4 N d^2 delta (per kv head)
  update backward           4 N d^2 linear (sigma(K) gM, V gM^T);
                            10 N d^2 + 2 d^3 delta (also sigma(K) M,
                            (Y / den) M^T, G_s, and (I - G_s) gM on the chain)
The arithmetic is fp32 throughout: products of two stored bf16 tensors run on
the bf16 matrix cores (a bf16 product is exact in fp32, and they accumulate in
fp32), the rest on the fp32 matrix cores and vector ALUs. The rate is priced
against the fp32 peak (157.3 TFLOP/s).
"""

from __future__ import annotations

import argparse
import json
import sys

from . import _lib

PEAK_FP32_TFLOPS = 157.3
SHAPES = {
    "llama3_8b_gqa": dict(B=1, Hq=32, Hkv=8, D=128, N=2048, L=32768, modes=("delta", "linear")),
    "llama300m_16k": dict(B=4, Hq=16, Hkv=16, D=64, N=2048, L=16384, modes=("delta",)),
    "stream_1m": dict(B=1, Hq=8, Hkv=8, D=128, N=2048, L=1048576, modes=("delta",)),
}


def algorithmic_flops(B, Hq, Hkv, D, N, L, mode):
    S = -(-L // N)
    per_q = 5.0 * N * N * D + 6.0 * N * D * D
    per_kv = (2.0 * N * D * D + 4.0 * N * D * D) if mode == "linear" else (
        4.0 * N * D * D + 10.0 * N * D * D + 2.0 * D ** 3)
    return S * (B * Hq * per_q + B * Hkv * per_kv)


def case(name, mode, steps, warmup=2, seed=0):
    import torch

    p = SHAPES[name]
    B, Hq, Hkv, D, N, L = p["B"], p["Hq"], p["Hkv"], p["D"], p["N"], p["L"]
    g = torch.Generator(device="cuda").manual_seed(seed)

    def randn(*s, scale=1.0):
        return (torch.randn(*s, generator=g, device="cuda") * scale).to(torch.bfloat16)

    q = randn(B, Hq, L, D, scale=D ** -0.5)
    k = randn(B, Hkv, L, D, scale=D ** -0.5)
    v = randn(B, Hkv, L, D, scale=D ** -0.5)
    d_out = randn(B, Hq, L, D)
    beta = torch.randn(Hq, generator=g, device="cuda")
    M0 = torch.zeros(B, Hkv, D, D, device="cuda")
    z0 = torch.full((B, Hkv, D), 2048.0, device="cuda")
    for _ in range(warmup):
        _lib.backward(q, k, v, beta, M0, z0, N, d_out, mode)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        grads = _lib.backward(q, k, v, beta, M0, z0, N, d_out, mode)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    finite = all(bool(torch.isfinite(t).all()) for t in grads)
    fl = algorithmic_flops(B, Hq, Hkv, D, N, L, mode)
    tf = fl / (ms * 1e-3) / 1e12
    return dict(workload=name, mode=mode, B=B, n_q_heads=Hq, n_kv_heads=Hkv, d=D, seg_len=N,
                seq_len=L, dtype="bf16 storage, fp32 arithmetic", steps=steps,
                ms_per_call=ms, tokens_per_s=B * L / (ms * 1e-3), gflop_per_call=fl / 1e9,
                tflops_algorithmic=tf, fp32_vector_peak_frac=tf / PEAK_FP32_TFLOPS,
                finite=finite)


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--shape", choices=sorted(SHAPES), action="append")
    args = ap.parse_args(argv)
    import torch

    if not torch.cuda.is_available():
        print("backward_bench needs a GPU", file=sys.stderr)
        return 2
    _lib.load()
    for name in args.shape or list(SHAPES):
        for mode in SHAPES[name]["modes"]:
            print(json.dumps(case(name, mode, args.steps, args.warmup)), flush=True)
    _lib.release_handles()
    return 0


if __name__ == "__main__":
    sys.exit(main())
