"""GPU parity of the Infini-attention block (infini_attn_block_forward with
three projection weights, and infini_attn_block_forward_qkv with the fused
[Wq|Wk|Wv] weight: rocBLAS projections into one row-major buffer that the
forward kernels read in place, the output projection) against the fp64
oracle, through the C ABI."""

import math

import numpy as np
import pytest

import synth
from parity import check, log, to_device, to_host64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import compressive_memory_transformers_segment_amd as ia
    ia.load()
    yield
    ia.release_handles()


def _store(a, dtype):
    x32 = np.asarray(a, dtype=np.float32)
    return synth.round_bf16_bits(x32) if dtype == "bf16" else x32


def block_case(seed, dtype, B, L, dm, Hq, Hkv, d, N, mode, fused=False):
    import torch
    import oracle
    import compressive_memory_transformers_segment_amd as ia

    rng = np.random.default_rng(seed)
    st = {n: _store(a, dtype) for n, a in dict(
        x=rng.standard_normal((B, L, dm)),
        wq=rng.standard_normal((dm, Hq * d)) / math.sqrt(dm),
        wk=rng.standard_normal((dm, Hkv * d)) / math.sqrt(dm),
        wv=rng.standard_normal((dm, Hkv * d)) / math.sqrt(dm),
        wo=rng.standard_normal((Hq * d, dm)) / math.sqrt(Hq * d)).items()}
    beta = rng.standard_normal(Hq).astype(np.float32)
    M0 = (0.05 * rng.standard_normal((B, Hkv, d, d))).astype(np.float32)
    z0 = rng.uniform(1.0, 20.0, (B, Hkv, d)).astype(np.float32)
    # The library takes weights [out, in]; the oracle takes them [in, out].
    dev = {n: to_device(a if n == "x" else np.ascontiguousarray(a.T), dtype)
           for n, a in st.items()}
    M = torch.from_numpy(M0).cuda()
    z = torch.from_numpy(z0).cuda()
    if fused:
        wqkv = to_device(np.ascontiguousarray(
            np.concatenate([st["wq"], st["wk"], st["wv"]], axis=1).T), dtype)
        y = ia.block_forward(dev["x"], None, None, None, dev["wo"],
                             torch.from_numpy(beta).cuda(), M, z, N, mode, n_q_heads=Hq,
                             n_kv_heads=Hkv, wqkv=wqkv)
    else:
        y = ia.block_forward(dev["x"], dev["wq"], dev["wk"], dev["wv"], dev["wo"],
                             torch.from_numpy(beta).cuda(), M, z, N, mode, n_q_heads=Hq,
                             n_kv_heads=Hkv)
    torch.cuda.synchronize()
    got = (to_host64(y, dtype), to_host64(M, "f32"), to_host64(z, "f32"))
    f64 = {n: synth.as_f64(a, dtype) for n, a in st.items()}
    ref = oracle.infini_block(f64["x"], f64["wq"], f64["wk"], f64["wv"], f64["wo"],
                              beta.astype(np.float64), M0.astype(np.float64),
                              z0.astype(np.float64), N, mode, Hq, Hkv, 1e-6)
    return got, ref


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mode", ["linear", "delta"])
@pytest.mark.parametrize("B,L,dm,Hq,Hkv,d,N", [(2, 300, 96, 4, 2, 32, 128),
                                               (1, 700, 160, 4, 1, 64, 256)])
def test_block_matches_oracle(dtype, mode, B, L, dm, Hq, Hkv, d, N, fused):
    """Small layers with d_model != Hq * d, grouped heads, ragged last segments."""
    log(f"block {dtype} {mode} B={B} L={L} dm={dm} Hq={Hq} Hkv={Hkv} d={d} N={N} fused={fused}")
    got, ref = block_case(1000 + L + d, dtype, B, L, dm, Hq, Hkv, d, N, mode, fused)
    check(f"block {dtype} {mode} y", got[0], ref[0], dtype)
    check(f"block {dtype} {mode} M", got[1], ref[1], dtype, state=True)
    check(f"block {dtype} {mode} z", got[2], ref[2], dtype, state=True)


@pytest.mark.parametrize("fused", [False, True])
def test_block_llama_width(fused):
    """A Llama-style layer at reduced length: d_model = 1024, 8 query heads,
    2 kv heads, d = 128, L = 2148 (a segment of 1024, another, and 100 rows),
    bf16, delta rule."""
    log(f"block llama width fused={fused}")
    got, ref = block_case(1100, "bf16", 1, 2148, 1024, 8, 2, 128, 1024, "delta", fused)
    check("block llama width y", got[0], ref[0], "bf16")
    check("block llama width M", got[1], ref[1], "bf16", state=True)
    check("block llama width z", got[2], ref[2], "bf16", state=True)


def test_block_rejects_bad_width():
    import torch
    import compressive_memory_transformers_segment_amd as ia
    x = torch.zeros((1, 8, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 1, 0, 64), dtype=torch.bfloat16, device="cuda")
    h = ia.handle_for(x.new_empty((1, 1, 0, 64)), k, seq_len=8)
    M = torch.zeros((1, 1, 64, 64), device="cuda")
    with pytest.raises(ia.InfiniAttnError) as ei:
        ia.infini_attn_block_forward(h, 0, x.data_ptr(), x.data_ptr(), x.data_ptr(), x.data_ptr(),
                                     x.data_ptr(), M.data_ptr(), M.data_ptr(), M.data_ptr(), 8, 0,
                                     x.data_ptr())
    assert ei.value.status == -1


def test_block_qkv_rejects_null_weight():
    import torch
    import compressive_memory_transformers_segment_amd as ia
    x = torch.zeros((1, 8, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 1, 0, 64), dtype=torch.bfloat16, device="cuda")
    h = ia.handle_for(x.new_empty((1, 1, 0, 64)), k, seq_len=8)
    M = torch.zeros((1, 1, 64, 64), device="cuda")
    with pytest.raises(ia.InfiniAttnError) as ei:
        ia.infini_attn_block_forward_qkv(h, 64, x.data_ptr(), 0, x.data_ptr(), M.data_ptr(),
                                         M.data_ptr(), M.data_ptr(), 8, 0, x.data_ptr())
    assert ei.value.status == -1
