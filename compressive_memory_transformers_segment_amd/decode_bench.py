"""Streaming-decode throughput on one GPU.

    python -m compressive_memory_transformers_segment_amd.decode_bench [--steps K]

One step is one infini_attn_decode call: C new rows per query head at position
n_past of the current segment, against a K/V cache holding that segment, plus
retrieval from (M, z). Shapes: the Llama-3-8B attention shape (B = 1, 32 query
heads, 8 kv heads, d = 128) and the streaming long-context shape (B = 1, 8
heads, d = 128), both with segments of 2048 rows and bf16 storage. Positions:
the last row of a segment (the most keys) and the middle, with C = 1 and a
16-row chunk. Inputs are seeded N(0, 1)/sqrt(d) values generated on the
device; (M, z) random with z > 0.

Each case prints one JSON line: microseconds per call (HIP events on the
launch stream around K back-to-back calls) through the C entry point with its
arguments marshalled once (`us_per_call`: the library's own cost per token)
and through the Python binding, which checks the tensors on every call
(`us_per_call_binding`: the host then sets the pace), decoded tokens/s
(B * C per call), and the algorithmic HBM bytes per call (the visible cache
rows of K and V, q, out, M, z) divided by the C-entry-point call time,
against the 8 TB/s HBM peak: decode reads every visible cache row once, so it
is bound by memory (and, at these sizes, by launch latency).
"""

from __future__ import annotations

import argparse
import json
import math
import sys

from . import _lib

PEAK_HBM_GBS = 8000.0
SHAPES = {"llama3_8b_gqa": (1, 32, 8, 128), "streaming_h8": (1, 8, 8, 128)}
CAP = 2048


def algorithmic_bytes(B, Hq, Hkv, D, C, n_past, elt=2):
    rows = n_past + C
    return (2 * B * Hkv * rows * D * elt + 2 * B * Hq * C * D * elt
            + B * Hkv * (D * D + D) * 4 + Hq * 4)


def case(shape, n_past, C, steps, warmup=20, seed=0):
    import torch

    B, Hq, Hkv, D = SHAPES[shape]
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(seed)

    def randn(*s):
        return (torch.randn(s, generator=g, device=dev) / math.sqrt(D)).to(torch.bfloat16)

    q = randn(B, Hq, C, D)
    kc, vc = randn(B, Hkv, CAP, D), randn(B, Hkv, CAP, D)
    M = 0.05 * torch.randn((B, Hkv, D, D), generator=g, device=dev)
    z = 1.0 + 49.0 * torch.rand((B, Hkv, D), generator=g, device=dev)
    beta = torch.randn((Hq,), generator=g, device=dev)
    out = torch.empty_like(q)

    def timed(call):
        for _ in range(warmup):
            call()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            call()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / steps

    us_binding = timed(lambda: _lib.decode(q, kc, vc, n_past, beta, M, z, out=out))
    # The same call with its arguments marshalled once (the handle is the
    # binding's cached one for these shapes and this stream).
    lib = _lib.load()
    h = _lib.handle_for(q, kc, 1e-6, seq_len=CAP)
    args = (h, q.data_ptr(), C, kc.data_ptr(), vc.data_ptr(), n_past, beta.data_ptr(),
            M.data_ptr(), z.data_ptr(), out.data_ptr())
    fn = lib.infini_attn_decode

    def direct():
        if fn(*args) != 0:
            raise RuntimeError("infini_attn_decode failed")

    us = timed(direct)
    if not bool(torch.isfinite(out.float()).all()):
        raise RuntimeError("non-finite output")
    nbytes = algorithmic_bytes(B, Hq, Hkv, D, C, n_past)
    gbs = nbytes / (us * 1e-6) / 1e9
    _lib.release_handles()
    return {
        "workload": shape, "batch": B, "n_q_heads": Hq, "n_kv_heads": Hkv, "d": D,
        "seg_len": CAP, "n_past": n_past, "new_rows": C, "steps": steps,
        "us_per_call": us, "us_per_call_binding": us_binding,
        "tokens_per_s": B * C / (us * 1e-6),
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": gbs / PEAK_HBM_GBS, "bytes_per_call": nbytes},
    }


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--steps", type=int, default=200)
    args = ap.parse_args(argv)
    import torch

    if not torch.cuda.is_available():
        print("decode_bench: no GPU visible", file=sys.stderr)
        return 2
    _lib.load()
    for shape in SHAPES:
        for n_past, C in ((CAP - 1, 1), (CAP // 2, 1), (CAP - 16, 16)):
            print(json.dumps(case(shape, n_past, C, args.steps)), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
