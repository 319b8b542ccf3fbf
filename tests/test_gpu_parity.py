"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle on
identical seeded inputs, element by element, at sizes the oracle finishes in
seconds that still span several tiles and a ragged tail."""

import numpy as np
import pytest

import synth
from parity import check, check_all, log, run_gpu, run_oracle

pytestmark = pytest.mark.gpu

INF = float("inf")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import compressive_memory_transformers_segment_amd as ia
    ia.load()
    yield
    ia.release_handles()


def test_tiny_f32_workload():
    """B=1, H=2, d=32, N=64, L=256, fp32, linear."""
    w = synth.WORKLOADS["tiny_f32"]
    inp = synth.generate(w)
    log(w.describe())
    check_all("tiny_f32", run_gpu(inp, "f32", w.seg_len, "linear"),
              run_oracle(inp, "f32", w.seg_len, "linear"), "f32")


@pytest.mark.parametrize("mode", ["linear", "delta"])
def test_small_200m_workload(mode):
    """B=2, H=8, d=64, N=64, 16 segments, bf16."""
    w = synth.WORKLOADS["small_200m"]
    inp = synth.generate(w)
    log(f"{w.describe()} {mode}")
    check_all(f"small_200m {mode}", run_gpu(inp, "bf16", w.seg_len, mode),
              run_oracle(inp, "bf16", w.seg_len, mode), "bf16")


# Several query tiles (128 rows), several key tiles (64 rows), a short last
# segment (700 = 300 + 300 + 100), grouped heads, a nonzero initial state, and
# gates at both limits next to finite ones.
RAGGED = dict(B=2, Hq=4, Hkv=2, L=700)
BETAS = np.array([-INF, -0.7, 1.3, INF], dtype=np.float32)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("mode", ["linear", "delta"])
def test_ragged_multi_tile(dtype, d, mode):
    inp = synth.random_case(100 + d, dk=d, dv=d, dtype=dtype, beta=BETAS, nonzero_state=True,
                            scale=1.5 / np.sqrt(d) * 4, **RAGGED)
    log(f"ragged {dtype} d={d} {mode}")
    check_all(f"ragged {dtype} d{d} {mode}", run_gpu(inp, dtype, 300, mode),
              run_oracle(inp, dtype, 300, mode), dtype)


# Query-head groups: 4 and 8 heads per kv head (four heads share each
# workgroup's K / V tiles), 6 (two), 3 (one).
@pytest.mark.parametrize("hq,hkv", [(4, 1), (8, 2), (6, 2), (3, 1)])
@pytest.mark.parametrize("d", [64, 128])
def test_grouped_heads(hq, hkv, d):
    betas = np.linspace(-2.0, 2.0, hq).astype(np.float32)
    inp = synth.random_case(300 + 10 * hq + d, B=1, Hq=hq, Hkv=hkv, L=700, dk=d, dv=d,
                            dtype="bf16", beta=betas, nonzero_state=True,
                            scale=1.5 / np.sqrt(d) * 4)
    log(f"grouped Hq={hq} Hkv={hkv} d={d}")
    check_all(f"grouped {hq}/{hkv} d{d}", run_gpu(inp, "bf16", 300, "delta"),
              run_oracle(inp, "bf16", 300, "delta"), "bf16")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_pure_branches(dtype):
    """beta = -inf isolates local attention; beta = +inf isolates retrieval."""
    inp = synth.random_case(7, B=1, Hq=2, Hkv=1, L=513, dk=64, dv=64, dtype=dtype,
                            nonzero_state=True, scale=0.5)
    for name, b in (("A_dot", -INF), ("A_mem", INF)):
        beta = np.full(2, b, dtype=np.float32)
        g = run_gpu(inp, dtype, 256, "delta", beta=beta)
        r = run_oracle(inp, dtype, 256, "delta", beta=beta)
        check(f"{dtype} {name}", g[0], r[0], dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_zero_state_first_segment_is_exactly_zero(dtype):
    """M0 = 0, z0 = 0 and beta = +inf: the first segment's output is bitwise 0."""
    inp = synth.random_case(8, B=1, Hq=2, Hkv=2, L=300, dk=64, dv=64, dtype=dtype, scale=0.7)
    out, _, _ = run_gpu(inp, dtype, 128, "delta", beta=np.full(2, INF, dtype=np.float32))
    assert np.all(out[:, :, :128] == 0.0) and not np.any(np.signbit(out[:, :, :128]))
    assert np.all(np.abs(out[:, :, 128:]).max(axis=-1) > 0.0)


@pytest.mark.parametrize("mode", ["linear", "delta"])
def test_split_calls_carry_state(mode):
    """forward(L) vs forward(L1) then forward(L - L1) with (M, z) passed back."""
    inp = synth.random_case(9, B=1, Hq=4, Hkv=2, L=640, dk=64, dv=64, dtype="bf16", scale=0.5)
    whole = run_gpu(inp, "bf16", 128, mode)
    L1 = 384
    first = dict(inp, q=inp["q"][:, :, :L1], k=inp["k"][:, :, :L1], v=inp["v"][:, :, :L1])
    o1, M1, z1 = run_gpu(first, "bf16", 128, mode)
    second = dict(inp, q=inp["q"][:, :, L1:], k=inp["k"][:, :, L1:], v=inp["v"][:, :, L1:],
                  M0=M1.astype(np.float32), z0=z1.astype(np.float32))
    o2, M2, z2 = run_gpu(second, "bf16", 128, mode)
    ref = run_oracle(inp, "bf16", 128, mode)
    check_all(f"split {mode}", (np.concatenate([o1, o2], axis=2), M2, z2), ref, "bf16")
    check_all(f"whole {mode}", whole, ref, "bf16")
    # fp32 state round trip: the two routes agree to fp32 rounding
    assert np.max(np.abs(M2 - whole[1])) <= 1e-5 * max(1.0, np.max(np.abs(whole[1])))


def test_bitwise_deterministic():
    inp = synth.random_case(10, B=1, Hq=4, Hkv=1, L=1000, dk=128, dv=128, dtype="bf16",
                            scale=0.6)
    a = run_gpu(inp, "bf16", 512, "delta")
    b = run_gpu(inp, "bf16", 512, "delta")
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("S", [7, 8, 9, 11, 17])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mode", ["linear", "delta"])
def test_segment_counts_around_the_scan_ring(S, d, mode):
    """Segment counts below, at and past the scan's register ring (3 steps for
    the delta rule, 8 for the linear rule): whole rounds, a remainder, both."""
    inp = synth.random_case(400 + 7 * S + d, B=1, Hq=2, Hkv=1, L=64 * S - 10, dk=d, dv=d,
                            dtype="bf16", nonzero_state=True, scale=1.5 / np.sqrt(d) * 4)
    log(f"S={S} d={d} {mode}")
    check_all(f"S={S} d{d} {mode}", run_gpu(inp, "bf16", 64, mode),
              run_oracle(inp, "bf16", 64, mode), "bf16")


@pytest.mark.parametrize("S,d,hq,hkv", [(63, 64, 2, 1), (64, 32, 2, 2), (100, 64, 4, 2),
                                         (131, 128, 2, 1), (200, 32, 2, 1)])
def test_long_chains_take_the_chunked_scan(S, d, hq, hkv):
    """Chains of 64 segments and more run the delta rule's recurrence as a
    chunked scan (per-chunk products in parallel, a chain over the chunks,
    then every chunk again from its start state): 63 segments (one chain),
    64 (chunks of 6, a short last chunk), 100, 131 and 200 segments, grouped
    heads and a short last segment, against the oracle's segment loop."""
    inp = synth.random_case(450 + S + d, B=1, Hq=hq, Hkv=hkv, L=16 * S - 5, dk=d, dv=d,
                            dtype="bf16", nonzero_state=True, scale=1.5 / np.sqrt(d) * 4)
    log(f"chunked scan S={S} d={d} Hq={hq} Hkv={hkv}")
    check_all(f"chunked S={S} d{d}", run_gpu(inp, "bf16", 16, "delta"),
              run_oracle(inp, "bf16", 16, "delta"), "bf16")


def test_long_chain_from_zero_state():
    """A chunked chain from M0 = 0, z0 = 0, where the first write divides by
    eps alone and the first chunk's product is huge, times a zero state."""
    inp = synth.random_case(470, B=1, Hq=2, Hkv=1, L=16 * 96, dk=64, dv=64, dtype="bf16",
                            scale=1.5 / 8.0 * 4)
    log("chunked scan from zero state")
    check_all("chunked zero state", run_gpu(inp, "bf16", 16, "delta"),
              run_oracle(inp, "bf16", 16, "delta"), "bf16")


@pytest.mark.parametrize("seg_len", [1, 5, 2000, 1 << 24, 2**31 - 1])
def test_segment_length_extremes(seg_len):
    """N = 1 (every row its own segment), an odd N, and N > L (one short
    segment), also N near the int32 limit."""
    inp = synth.random_case(11, B=1, Hq=2, Hkv=1, L=200, dk=32, dv=32, dtype="bf16",
                            nonzero_state=True, scale=0.5)
    check_all(f"N={seg_len}", run_gpu(inp, "bf16", seg_len, "delta"),
              run_oracle(inp, "bf16", seg_len, "delta"), "bf16")


def test_empty_sequence_is_a_no_op():
    import torch
    import compressive_memory_transformers_segment_amd as ia
    q = torch.empty((1, 2, 0, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.empty((1, 1, 0, 64), dtype=torch.bfloat16, device="cuda")
    M = torch.randn((1, 1, 64, 64), device="cuda")
    z = torch.rand((1, 1, 64), device="cuda")
    M0, z0 = M.clone(), z.clone()
    out = ia.forward(q, k, k, torch.zeros(2, device="cuda"), M, z, 64, "delta")
    torch.cuda.synchronize()
    assert out.shape == (1, 2, 0, 64)
    assert torch.equal(M, M0) and torch.equal(z, z0)


def test_invalid_arguments_are_rejected_before_launch():
    import torch
    import compressive_memory_transformers_segment_amd as ia
    inp = synth.random_case(12, B=1, Hq=2, Hkv=1, L=64, dk=64, dv=64, dtype="bf16")
    q = torch.zeros((1, 2, 64, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 1, 64, 64), dtype=torch.bfloat16, device="cuda")
    M = torch.zeros((1, 1, 64, 64), device="cuda")
    z = torch.zeros((1, 1, 64), device="cuda")
    beta = torch.zeros(2, device="cuda")
    with pytest.raises(ia.InfiniAttnError) as ei:
        ia.forward(q, k, k, beta, M, z, 0, "linear")
    assert ei.value.status == -1
    h = ia.handle_for(q, k)
    with pytest.raises(ia.InfiniAttnError) as ei:
        ia.infini_attn_forward(h, q.data_ptr() + 2, k.data_ptr(), k.data_ptr(), beta.data_ptr(),
                               M.data_ptr(), z.data_ptr(), 64, 0, q.data_ptr())
    assert ei.value.status == -1
    with pytest.raises(ia.InfiniAttnError) as ei:
        ia.infini_attn_forward(h, q.data_ptr(), k.data_ptr(), k.data_ptr(), beta.data_ptr(),
                               M.data_ptr(), z.data_ptr(), 64, 3, q.data_ptr())
    assert ei.value.status == -1
    assert inp["q"].shape == (1, 2, 64, 64)


@pytest.mark.parametrize("d", [64, 128])
def test_one_long_segment_is_full_causal_attention(d):
    """N = L: one segment of 3000 rows (47 key tiles, a ragged tail), the
    full-causal case the scaling sweep uses as its quadratic reference."""
    inp = synth.random_case(500 + d, B=1, Hq=2, Hkv=1, L=3000, dk=d, dv=d, dtype="bf16",
                            nonzero_state=True, scale=1.5 / np.sqrt(d) * 4)
    log(f"one segment L=N=3000 d={d}")
    check_all(f"N=L d{d}", run_gpu(inp, "bf16", 3000, "delta"),
              run_oracle(inp, "bf16", 3000, "delta"), "bf16")
