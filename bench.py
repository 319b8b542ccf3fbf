"""Throughput of the Infini-attention forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--mode delta|linear]

One step is one forward pass of the whole path (segment scan, then the fused
per-segment kernel) over one batch of synthetic, seeded input already resident
in HBM. Prints ONE JSON line on stdout; progress goes to stderr.

Default workload: the Llama-3-8B attention shape (B=1, 32 query heads, 8 kv
heads, d=128, segments of 2048 rows, L=32768, bf16 storage).
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Infini-attn fwd tokens/sec on 1 MI355X; % MFMA bf16 peak; HBM GB/s"
PEAK_BF16_TFLOPS = 2516.6  # 256 CU x 4096 bf16 FLOP/clk x 2.4 GHz (dense MFMA)
PEAK_F32_VALU_TFLOPS = 157.3  # published fp32 vector peak (packed FMA, 256 CU at 2.4 GHz)
PEAK_HBM_GBS = 8000.0


def log(msg: str) -> None:
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def segment_rows(L: int, N: int):
    return [min(N, L - a) for a in range(0, L, N)]


def work_counts(w, mode: str) -> dict:
    """Algorithmic FLOPs and bytes of one forward pass.

    Fused kernel, per (query head, segment of n rows): local causal attention
    over n(n+1)/2 (query, key) pairs, 2d FLOPs each for Q K^T and for P V,
    plus 2 n d^2 for the retrieval sigma(Q) M. Scan, per (kv head, segment):
    2 n d^2 (sigma(K)^T V) for the linear rule, 4 n d^2 with the delta rule's
    retrieval. Softmax, feature-map and normaliser arithmetic is not counted.
    Bytes: Q, K, V read once and out written once (storage dtype), plus the
    fp32 state read and written once.
    """
    d = w.d
    el = 2 if w.dtype == "bf16" else 4
    rows = segment_rows(w.seq_len, w.seg_len)
    attn = sum(4 * d * n * (n + 1) // 2 for n in rows)
    retr = sum(2 * n * d * d for n in rows)
    fused = w.batch * w.n_q_heads * (attn + retr)
    per_upd = (4 if mode == "delta" else 2) * d * d
    scan = w.batch * w.n_kv_heads * sum(per_upd * n for n in rows)
    qo = 2 * w.batch * w.n_q_heads * w.seq_len * d * el
    kv = 2 * w.batch * w.n_kv_heads * w.seq_len * d * el
    state = 2 * w.batch * w.n_kv_heads * (d * d + d) * 4
    return dict(fused_flops=fused, scan_flops=scan, total_flops=fused + scan,
                bytes=qo + kv + state, fused_bytes=qo + kv)


def fused_kernel_name(w) -> str:
    if w.dtype != "bf16":
        return f"fused_f32_kernel<{w.d}>"
    g = w.n_q_heads // w.n_kv_heads
    return f"fused_bf16_kernel<{w.d}, {4 if g % 4 == 0 else 2 if g % 2 == 0 else 1}>"


def host_info() -> dict:
    """CPU model, BLAS library and its thread count on this host."""
    import numpy as np
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    a = np.ones((64, 64))
    _ = a @ a  # loads the BLAS library so that threadpoolctl sees it
    blas, threads = "unknown", 1
    try:
        from threadpoolctl import threadpool_info
        infos = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if infos:
            blas = f"{infos[0].get('internal_api')} {infos[0].get('version')}"
            threads = max(i.get("num_threads", 1) for i in infos)
    except Exception:  # noqa: BLE001
        pass
    return {"cpu_model": model, "blas": blas, "blas_threads": threads,
            "cpus_visible": len(os.sched_getaffinity(0))}


def cpu_baseline(w, inp, mode: str, budget_s: float) -> dict:
    """The fp64 oracle on the host cores, on the first segments of the same
    workload (all batch entries and heads), scaled to tokens/s."""
    import numpy as np

    import oracle
    import synth

    info = host_info()
    N = w.seg_len

    def run(n_seg: int) -> float:
        L = min(n_seg * N, w.seq_len)
        q = synth.as_f64(inp["q"][:, :, :L], w.dtype)
        k = synth.as_f64(inp["k"][:, :, :L], w.dtype)
        v = synth.as_f64(inp["v"][:, :, :L], w.dtype)
        t0 = time.perf_counter()
        oracle.infini_attention(q, k, v, inp["beta"].astype(np.float64),
                                inp["M0"].astype(np.float64), inp["z0"].astype(np.float64), N,
                                mode, float(inp["eps"]))
        return time.perf_counter() - t0

    t1 = run(1)
    n = max(1, min(w.n_segments, int(budget_s / max(t1, 1e-3))))
    reps = 1
    if n > 1:
        t = run(n)
    else:
        n, t = 1, t1
    if n == w.n_segments and t < 0.5 * budget_s:
        # The whole workload is a short sample: repeat it to fill the budget.
        reps = max(1, int(budget_s / max(t, 1e-4)))
        t = sum(run(n) for _ in range(reps))
    tokens = w.batch * min(n * N, w.seq_len)
    return {"value": reps * tokens / t, "unit": "tokens/s", "cores": info["blas_threads"],
            "kind": "oracle",
            "sample": f"first {n} of {w.n_segments} segments ({tokens} tokens, all "
                      f"{w.batch * w.n_q_heads} query heads) x {reps}, {mode} rule, "
                      f"fp64 numpy; {t:.2f} s",
            "cpu_model": info["cpu_model"], "blas": info["blas"],
            "cpus_visible": info["cpus_visible"]}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama3_8b_gqa")
    ap.add_argument("--mode", default="delta", choices=["linear", "delta"])
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="after the timed run, copy this many bytes device-to-device (a plain "
                         "copy kernel of known size, used to calibrate HBM byte counters)")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: --gpus {args.gpus} is not supported "
              "(the Infini-attention forward here is a single-GPU kernel pair; heads would "
              "shard across GPUs with no communication, see the design notes).",
              file=sys.stderr)
        return 2
    rank = int(os.environ.get("RANK", "0"))

    import numpy as np
    import torch

    import compressive_memory_transformers_segment_amd as ia
    import synth

    from compressive_memory_transformers_segment_amd import traffic as traffic_mod

    w = synth.WORKLOADS[args.workload]
    ia.load()
    log(f"generating {w.describe()}")
    t0 = time.perf_counter()
    inp = synth.generate(w)
    log(f"inputs ready in {time.perf_counter() - t0:.1f} s")
    dev = torch.device("cuda:0")

    def up(a):
        if w.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
                torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    q, k, v = up(inp["q"]), up(inp["k"]), up(inp["v"])
    beta = torch.from_numpy(inp["beta"]).to(dev)
    M0 = torch.from_numpy(inp["M0"]).to(dev)
    z0 = torch.from_numpy(inp["z0"]).to(dev)
    M, z = M0.clone(), z0.clone()
    out = torch.empty((w.batch, w.n_q_heads, w.seq_len, w.d), dtype=q.dtype, device=dev)
    h = ia.handle_for(q, k, w.eps)
    n_ev = args.warmup + args.steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n_ev)]

    def step(i):
        # Every step starts from the workload's initial state (reset outside the
        # events); the events bracket the forward call on the stream it runs on.
        M.copy_(M0)
        z.copy_(z0)
        ev[i][0].record()
        ia.forward(q, k, v, beta, M, z, w.seg_len, args.mode, out=out, eps=w.eps)
        ev[i][1].record()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ia.infini_attn_set_timing(h, True)
    ia.infini_attn_get_timing(h)  # clear
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.warmup, n_ev):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    calls, scan_ms, fused_ms = ia.infini_attn_get_timing(h)
    ia.infini_attn_set_timing(h, False)
    assert calls == args.steps, (calls, args.steps)
    if not bool(torch.isfinite(out.float()).all()):
        log("ERROR: non-finite output")
        return 1
    step_ms = sorted(ev[i][0].elapsed_time(ev[i][1]) for i in range(args.warmup, n_ev))
    med_ms = step_ms[len(step_ms) // 2] if len(step_ms) % 2 else 0.5 * (
        step_ms[len(step_ms) // 2 - 1] + step_ms[len(step_ms) // 2])

    wc = work_counts(w, args.mode)
    tokens = w.batch * w.seq_len
    fused_avg_s = fused_ms / calls / 1e3
    scan_avg_s = scan_ms / calls / 1e3
    achieved = wc["fused_flops"] / fused_avg_s / 1e12
    kname = fused_kernel_name(w)
    counted = traffic_mod.load(w.name, args.mode)
    kernel_traffic = None
    hbm_counters = None
    traffic_ratio = None
    if counted is not None:
        if kname in counted:
            kernel_traffic = counted[kname]["fetch"] + counted[kname]["write"]
        pass_bytes = sum(c["fetch"] + c["write"] for c in counted.values())
        hbm_counters = pass_bytes / (med_ms / 1e3) / 1e9
        traffic_ratio = pass_bytes / wc["bytes"]
    bf16 = w.dtype == "bf16"
    peak = PEAK_BF16_TFLOPS if bf16 else PEAK_F32_VALU_TFLOPS
    tflops = wc["total_flops"] / (med_ms / 1e3) / 1e12
    result = {
        "metric": METRIC,
        "value": tokens / (med_ms / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": med_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1)/sqrt(d) q, k, v; see synth/)",
        "config": {"workload": w.name, "batch": w.batch, "n_q_heads": w.n_q_heads,
                   "n_kv_heads": w.n_kv_heads, "d": w.d, "seg_len": w.seg_len,
                   "seq_len": w.seq_len, "segments": w.n_segments, "update": args.mode},
        "timing": {"ms_per_step_median": med_ms, "ms_per_step_min": step_ms[0],
                   "ms_per_step_max": step_ms[-1],
                   "wall_ms_per_step_with_state_reset": elapsed * 1e3 / args.steps},
        "tflops_algorithmic": tflops,
        "mfma_bf16_peak_frac": tflops / PEAK_BF16_TFLOPS,
        "hbm_gbs_algorithmic": wc["bytes"] / (med_ms / 1e3) / 1e9,
        "hbm_gbs_counters": hbm_counters,
        "hbm_traffic_over_algorithmic": traffic_ratio,
        "kernels_ms": {"segment_scan": scan_avg_s * 1e3, "fused_attention": fused_avg_s * 1e3},
        "roofline": {
            "kernel": kname,
            "bound": "mfma" if bf16 else "alu",
            "achieved": achieved,
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": achieved / peak,
            "traffic": kernel_traffic,
            "flops_per_launch": wc["fused_flops"],
        },
    }
    if rank == 0 and not args.no_cpu_baseline:
        log("timing the fp64 oracle on the host cores")
        result["cpu_baseline"] = cpu_baseline(w, inp, args.mode, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    if args.copy_bytes > 0:
        src = torch.empty(args.copy_bytes, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_calibration_bytes"] = args.copy_bytes
    ia.release_handles()
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
