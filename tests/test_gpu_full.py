"""GPU parity at the full workload sizes, in the launch configuration bench.py
times. The oracle recomputes the whole (M, z) chain of every kv head (so the
final state is compared element by element) and, on sampled rows of every
query head, the output one row at a time: local attention from the
definition and retrieval from the oracle's own state before that row's
segment."""

import numpy as np
import pytest

import oracle
import synth
from parity import check, log, to_device, to_host64

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import compressive_memory_transformers_segment_amd as ia
    ia.load()
    yield
    ia.release_handles()
    torch.cuda.empty_cache()


def sample_plan(w, rng):
    """Every (batch, query head) pair; four segments (first, second, middle,
    last); rows at the boundaries of the kernel's 32-row wave strips and 64-
    and 256-row work items, the segment's last row, and six random ones."""
    S = w.n_segments
    segs = sorted({0, 1, S // 2, S - 1})
    heads = [(b, h) for b in range(w.batch) for h in range(w.n_q_heads)]
    edges = {0, 1, 31, 32, 63, 64, 127, 128, 129, 255, 256, w.seg_len - 1}
    rows = sorted({r for r in edges if r < w.seg_len} |
                  set(int(x) for x in rng.integers(0, w.seg_len, 6)))
    return segs, heads, rows


def run_full(name, mode):
    import torch
    import compressive_memory_transformers_segment_amd as ia

    w = synth.WORKLOADS[name]
    log(f"generating {w.describe()} {mode}")
    inp = synth.generate(w)
    q, k, v = (to_device(inp[x], w.dtype) for x in ("q", "k", "v"))
    beta = torch.from_numpy(inp["beta"]).cuda()
    M = torch.from_numpy(inp["M0"]).cuda()
    z = torch.from_numpy(inp["z0"]).cuda()
    log("gpu forward")
    out = ia.forward(q, k, v, beta, M, z, w.seg_len, mode, eps=w.eps)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out.float()).all())
    rng = np.random.default_rng(123)
    segs, heads, rows = sample_plan(w, rng)
    N, L, d = w.seg_len, w.seq_len, w.d
    pos = np.array([s * N + r for s in segs for r in rows if s * N + r < L])
    pos_t = torch.from_numpy(pos).cuda()
    got_rows = to_host64(torch.stack([out[b, h].index_select(0, pos_t) for b, h in heads]),
                         w.dtype)
    M_gpu, z_gpu = to_host64(M, "f32"), to_host64(z, "f32")
    del q, k, v, out
    torch.cuda.empty_cache()

    log("oracle state chain")
    up = lambda a: synth.as_f64(a, w.dtype)
    g = w.n_q_heads // w.n_kv_heads
    need = {(b, h // g) for b, h in heads}
    M_ref = np.empty_like(M_gpu)
    z_ref = np.empty_like(z_gpu)
    states = {}
    for b in range(w.batch):
        for j in range(w.n_kv_heads):
            keep = (b, j) in need
            Mf, zf, st = oracle.memory_chain(inp["k"][b, j], inp["v"][b, j],
                                             inp["M0"][b, j].astype(np.float64),
                                             inp["z0"][b, j].astype(np.float64), N, mode,
                                             w.eps, keep_states=keep, upcast=up)
            M_ref[b, j], z_ref[b, j] = Mf, zf
            if keep:
                states[(b, j)] = st
    check(f"{name} {mode} M", M_gpu, M_ref, w.dtype, state=True)
    check(f"{name} {mode} z", z_gpu, z_ref, w.dtype, state=True)

    log("oracle sampled rows")
    gam = oracle.gate_value(inp["beta"].astype(np.float64))
    ref_rows = np.empty_like(got_rows)
    for hi, (b, h) in enumerate(heads):
        j = oracle.kv_head_of(h, w.n_q_heads, w.n_kv_heads)
        col = 0
        for s in segs:
            a, e = s * N, min(s * N + N, L)
            K, V = up(inp["k"][b, j, a:e]), up(inp["v"][b, j, a:e])
            sel = [r for r in rows if a + r < e]
            qr = up(inp["q"][b, h, [a + r for r in sel]])
            adot = oracle.local_causal_attention_rows(qr, np.array(sel), K, V)
            Mp, zp = states[(b, j)][s]
            amem = oracle.memory_retrieval(qr, Mp, zp, w.eps)
            ref_rows[hi, col:col + len(sel)] = gam[h] * amem + (1 - gam[h]) * adot
            col += len(sel)
    check(f"{name} {mode} out (sampled {ref_rows.shape[0]}x{ref_rows.shape[1]} rows)",
          got_rows, ref_rows, w.dtype)


@pytest.mark.timeout(400)
def test_llama300m_16k_delta():
    run_full("llama300m_16k", "delta")


@pytest.mark.timeout(400)
@pytest.mark.parametrize("mode", ["linear", "delta"])
def test_llama3_8b_gqa(mode):
    run_full("llama3_8b_gqa", mode)


@pytest.mark.timeout(900)
def test_stream_1m_delta():
    run_full("stream_1m", "delta")
