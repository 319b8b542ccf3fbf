"""Forward time and device memory of Infini-attention against sequence length.

    python -m compressive_memory_transformers_segment_amd.scaling [--mode delta|linear]
        [--lengths 2048,8192,...] [--seg-len 2048] [--quadratic-max L]

The linear-cost claim ("Как работает Infini-attention (Google, 2024) для
бесконечного контекста?", section 4 on why the cost is linear, and its
closing project outline, which times forward passes against plain attention
at lengths from 1K tokens up): with a fixed segment length N the work per
token is constant (one N-row causal window plus one retrieval from a d x d
memory), so forward time grows linearly in L, and the state carried between
segments is one (M, z) per head whatever L is. The quadratic reference is
the same library call with N = L: one segment, i.e. plain causal attention
over the whole sequence (plus a retrieval from the initial state).

The shape is the streaming long-context one (B = 1, 8 heads, d = 128, bf16
storage, fp32 state), with seeded N(0, 1)/sqrt(d) inputs generated on the
device (torch's Philox generator), beta ~ N(0, 1) and a zero initial state.
Each point prints one JSON line: milliseconds per forward (wall clock over
the timed calls, and the library's per-kernel HIP-event times), tokens/s,
and the device bytes the call touches (caller tensors and the library's
workspace).
"""

from __future__ import annotations

import argparse
import json
import math
import sys
import time

from . import _lib

DEFAULT_LENGTHS = (2048, 8192, 32768, 131072, 524288, 1048576)


def _time_calls(q, k, v, beta, M, z, seg_len, mode, min_seconds, min_steps):
    import torch

    h = _lib.handle_for(q, k)
    out = torch.empty_like(q)
    _lib.forward(q, k, v, beta, M, z, seg_len, mode, out=out)  # warm-up (allocates workspace)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    _lib.forward(q, k, v, beta, M, z, seg_len, mode, out=out)
    torch.cuda.synchronize()
    one = time.perf_counter() - t0
    steps = max(min_steps, int(math.ceil(min_seconds / max(one, 1e-6))))
    _lib.infini_attn_set_timing(h, True)
    _lib.infini_attn_get_timing(h)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        _lib.forward(q, k, v, beta, M, z, seg_len, mode, out=out)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    calls, scan_ms, fused_ms = _lib.infini_attn_get_timing(h)
    _lib.infini_attn_set_timing(h, False)
    if calls != steps:
        raise RuntimeError(f"timed {calls} calls, expected {steps}")
    if not bool(torch.isfinite(out.float()).all()):
        raise RuntimeError("non-finite output")
    return steps, elapsed * 1e3 / steps, scan_ms / calls, fused_ms / calls


def point(L, seg_len, mode, heads=8, d=128, seed=0, min_seconds=0.3, min_steps=3):
    """Time one (L, N) point; returns a dict (one JSON line)."""
    import torch

    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(seed)

    def randn(*shape):
        return (torch.randn(shape, generator=g, device=dev) / math.sqrt(d)).to(torch.bfloat16)

    q, k, v = randn(1, heads, L, d), randn(1, heads, L, d), randn(1, heads, L, d)
    beta = torch.randn((heads,), generator=g, device=dev)
    M = torch.zeros((1, heads, d, d), device=dev)
    z = torch.zeros((1, heads, d), device=dev)
    desc = _lib.make_desc(1, heads, heads, L, d, d, _lib.BF16)
    ws = _lib.infini_attn_workspace_size(desc, seg_len)
    steps, ms, scan_ms, fused_ms = _time_calls(q, k, v, beta, M, z, seg_len, mode, min_seconds,
                                               min_steps)
    tensor_bytes = 4 * q.numel() * 2 + (M.numel() + z.numel() + beta.numel()) * 4
    res = {
        "L": L, "seg_len": seg_len, "segments": -(-L // seg_len), "update": mode,
        "heads": heads, "d": d, "steps": steps, "ms_per_forward": ms,
        "scan_ms": scan_ms, "fused_ms": fused_ms, "tokens_per_s": L / ms * 1e3,
        "us_per_1k_tokens": ms * 1e6 / L,
        "state_bytes": (M.numel() + z.numel()) * 4,
        "tensor_bytes": tensor_bytes, "workspace_bytes": ws,
    }
    _lib.release_handles()
    del q, k, v, M, z, beta
    torch.cuda.empty_cache()
    return res


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--mode", default="delta", choices=["linear", "delta"])
    ap.add_argument("--seg-len", type=int, default=2048)
    ap.add_argument("--lengths", default=",".join(str(x) for x in DEFAULT_LENGTHS))
    ap.add_argument("--quadratic-max", type=int, default=1048576,
                    help="largest L timed with N = L (one causal segment)")
    args = ap.parse_args(argv)
    import torch

    if not torch.cuda.is_available():
        print("scaling: no GPU visible", file=sys.stderr)
        return 2
    _lib.load()
    for L in (int(x) for x in args.lengths.split(",")):
        print(json.dumps(dict(kind="infini", **point(L, args.seg_len, args.mode))), flush=True)
        if L <= args.quadratic_max:
            print(json.dumps(dict(kind="full_causal", **point(L, L, args.mode, min_steps=2))),
                  flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
