"""Throughput of the whole Infini-attention block on one GPU.

    python -m compressive_memory_transformers_segment_amd.block_bench [--steps K]
        [--mode delta|linear] [--weights fused|separate]

One step is one block call at the Llama-3-8B layer shape: x [1, 32768, 4096]
bf16, 32 query heads and 8 kv heads of d = 128 (weights [out, in]: wq [4096,
4096], wk / wv [1024, 4096], wo [4096, 4096]), segments of 2048 rows; with
fused weights (the default) infini_attn_block_forward_qkv takes Wq, Wk, Wv
stacked, [6144, 4096], and projects with one GEMM, with separate ones
infini_attn_block_forward runs one GEMM per weight.
Inputs are seeded on the device: x ~ N(0, 1), weights ~ N(0, 1/fan_in),
beta ~ N(0, 1), zero initial state. Prints one JSON line: ms per block,
tokens/s, and the algorithmic TFLOP/s of the block (projections, attention,
retrieval and memory update) against the bf16 MFMA peak.
"""

from __future__ import annotations

import argparse
import json
import math
import sys

from . import _lib

PEAK_BF16_TFLOPS = 2516.6


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--mode", default="delta", choices=["linear", "delta"])
    ap.add_argument("--weights", default="fused", choices=["fused", "separate"])
    args = ap.parse_args(argv)
    import torch

    if not torch.cuda.is_available():
        print("block_bench: no GPU visible", file=sys.stderr)
        return 2
    _lib.load()
    B, L, dm, Hq, Hkv, D, N = 1, 32768, 4096, 32, 8, 128, 2048
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(0)

    def rnd(*shape, scale=1.0):
        return (scale * torch.randn(shape, generator=g, device=dev)).to(torch.bfloat16)

    x = rnd(B, L, dm)
    # Weights [out, in], as a linear layer keeps them.
    wq, wk, wv = (rnd(n * D, dm, scale=1 / math.sqrt(dm)) for n in (Hq, Hkv, Hkv))
    wo = rnd(dm, Hq * D, scale=1 / math.sqrt(Hq * D))
    wqkv = torch.cat([wq, wk, wv], dim=0).contiguous() if args.weights == "fused" else None
    beta = torch.randn((Hq,), generator=g, device=dev)
    M = torch.zeros((B, Hkv, D, D), device=dev)
    z = torch.zeros((B, Hkv, D), device=dev)
    y = torch.empty_like(x)

    def step():
        if wqkv is not None:
            _lib.block_forward(x, None, None, None, wo, beta, M, z, N, args.mode, n_q_heads=Hq,
                               n_kv_heads=Hkv, out=y, wqkv=wqkv)
        else:
            _lib.block_forward(x, wq, wk, wv, wo, beta, M, z, N, args.mode, n_q_heads=Hq,
                               n_kv_heads=Hkv, out=y)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    if not bool(torch.isfinite(y.float()).all()):
        print("block_bench: non-finite output", file=sys.stderr)
        return 1
    S = L // N
    proj = 2 * B * L * dm * (Hq + 2 * Hkv) * D + 2 * B * L * Hq * D * dm
    attn = B * Hq * S * (4 * D * N * (N + 1) / 2 + 2 * N * D * D)
    scan = B * Hkv * S * 2 * N * D * D * (2 if args.mode == "delta" else 1)
    flops = proj + attn + scan
    res = {
        "workload": "llama3_8b_layer", "batch": B, "seq_len": L, "d_model": dm,
        "n_q_heads": Hq, "n_kv_heads": Hkv, "d": D, "seg_len": N, "update": args.mode,
        "weights": args.weights,
        "steps": args.steps, "ms_per_block": ms, "tokens_per_s": B * L / (ms * 1e-3),
        "flops": {"projections": proj, "attention_retrieval": attn, "memory_update": scan},
        "tflops_algorithmic": flops / (ms * 1e-3) / 1e12,
        "mfma_bf16_peak_frac": flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
    }
    _lib.release_handles()
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
