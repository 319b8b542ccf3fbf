"""Helpers for GPU-vs-oracle parity: device transfer of stored inputs, running
both sides on the same seeded tensors, and the error metrics.

Tolerances (fp32 storage): normwise max relative error max|g - o| / max|o| <= 1e-4.
Tolerances (bf16 storage, fp32 accumulation): relative L2 error <= 2e-2 and
max absolute error <= 5e-2 on out; on the fp32 state (M, z), whose entries
grow with the number of rows written (z reaches about 1e6 after 2^20 rows,
where one fp32 ulp is 0.125), the absolute bound is scaled by max(1, max|o|).
"""

from __future__ import annotations

import sys
import time

import numpy as np

import synth

F32_TOL = 1e-4
BF16_REL_L2 = 2e-2
BF16_MAX_ABS = 5e-2


def log(msg: str) -> None:
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def to_device(arr: np.ndarray, dtype: str, device="cuda"):
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.to(device)


def to_host64(t, dtype: str) -> np.ndarray:
    import torch
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return synth.as_f64(t.view(torch.int16).numpy().view(np.uint16), "bf16")
    return t.numpy().astype(np.float64)


def run_gpu(inp: dict, dtype: str, seg_len: int, mode: str, beta=None):
    """One forward through the C ABI; returns (out, M, z) as fp64 numpy arrays."""
    import torch
    import compressive_memory_transformers_segment_amd as ia

    q = to_device(inp["q"], dtype)
    k = to_device(inp["k"], dtype)
    v = to_device(inp["v"], dtype)
    b = inp["beta"] if beta is None else np.asarray(beta, dtype=np.float32)
    bt = torch.from_numpy(np.ascontiguousarray(b, dtype=np.float32)).cuda()
    M = torch.from_numpy(np.ascontiguousarray(inp["M0"], dtype=np.float32)).cuda()
    z = torch.from_numpy(np.ascontiguousarray(inp["z0"], dtype=np.float32)).cuda()
    out = ia.forward(q, k, v, bt, M, z, seg_len, mode, eps=float(inp["eps"]))
    torch.cuda.synchronize()
    return to_host64(out, dtype), to_host64(M, "f32"), to_host64(z, "f32")


def run_oracle(inp: dict, dtype: str, seg_len: int, mode: str, beta=None):
    import oracle
    b = inp["beta"] if beta is None else np.asarray(beta, dtype=np.float32)
    return oracle.infini_attention(synth.as_f64(inp["q"], dtype), synth.as_f64(inp["k"], dtype),
                                   synth.as_f64(inp["v"], dtype), b.astype(np.float64),
                                   inp["M0"].astype(np.float64), inp["z0"].astype(np.float64),
                                   seg_len, mode, float(inp["eps"]))


def errors(got: np.ndarray, ref: np.ndarray) -> dict:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    diff = got - ref
    ref_max = float(np.max(np.abs(ref))) if ref.size else 0.0
    ref_l2 = float(np.linalg.norm(ref))
    return dict(
        max_abs=float(np.max(np.abs(diff))) if diff.size else 0.0,
        rel_l2=float(np.linalg.norm(diff) / ref_l2) if ref_l2 > 0 else float(np.linalg.norm(diff)),
        max_rel=float(np.max(np.abs(diff)) / ref_max) if ref_max > 0 else float(np.max(np.abs(diff), initial=0.0)),
        ref_max=ref_max,
        finite=bool(np.all(np.isfinite(got))),
    )


def check(name: str, got, ref, dtype: str, state: bool = False) -> dict:
    e = errors(got, ref)
    log(f"{name}: {e}")
    assert e["finite"], f"{name}: non-finite values"
    if dtype == "f32":
        assert e["max_rel"] <= F32_TOL, f"{name}: fp32 max relative error {e['max_rel']:.3e}"
    else:
        assert e["rel_l2"] <= BF16_REL_L2, f"{name}: relative L2 error {e['rel_l2']:.3e}"
        bound = BF16_MAX_ABS * (max(1.0, e["ref_max"]) if state else 1.0)
        assert e["max_abs"] <= bound, f"{name}: max abs error {e['max_abs']:.3e} > {bound:.3e}"
    return e


def check_all(tag: str, gpu, ref, dtype: str) -> None:
    check(f"{tag} out", gpu[0], ref[0], dtype)
    check(f"{tag} M", gpu[1], ref[1], dtype, state=True)
    check(f"{tag} z", gpu[2], ref[2], dtype, state=True)
