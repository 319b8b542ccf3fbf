"""GPU test of the allocation-free decode (infini_attn_decode_noalloc), called
through the C ABI: on the same inputs it must give the output of
infini_attn_decode (whose parity with the oracle the decode tests establish),
bit for bit, since both run the same kernels; on two calls in a row, the second
with a smaller input, so stale partials of the first call in the shared scratch
array cannot leak into the second; and a request larger than the fixed scratch
is rejected before anything is enqueued."""

import ctypes

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


def _inputs(seed, dtype, B, Hq, Hkv, cap, d, n_past, n_new):
    import torch
    c = synth.random_case(seed, B=B, Hq=Hq, Hkv=Hkv, L=cap, dk=d, dv=d, dtype=dtype,
                          nonzero_state=True, scale=1.5 / np.sqrt(d) * 4)
    q = to_device(c["q"][:, :, n_past:n_past + n_new].copy(), dtype)
    kc = to_device(c["k"], dtype)
    vc = to_device(c["v"], dtype)
    beta = torch.from_numpy(np.ascontiguousarray(c["beta"], dtype=np.float32)).cuda()
    M = torch.from_numpy(np.ascontiguousarray(c["M0"], dtype=np.float32)).cuda()
    z = torch.from_numpy(np.ascontiguousarray(c["z0"], dtype=np.float32)).cuda()
    return q, kc, vc, beta, M, z


def _call(fn_name, h, q, kc, vc, n_past, beta, M, z, out):
    lib = __import__("compressive_memory_transformers_segment_amd")._lib.load()
    fn = getattr(lib, fn_name)
    return fn(ctypes.c_void_p(h), ctypes.c_void_p(q.data_ptr()), q.shape[2],
              ctypes.c_void_p(kc.data_ptr()), ctypes.c_void_p(vc.data_ptr()), n_past,
              ctypes.c_void_p(beta.data_ptr()), ctypes.c_void_p(M.data_ptr()),
              ctypes.c_void_p(z.data_ptr()), ctypes.c_void_p(out.data_ptr()))


def _both(seed, dtype, B, Hq, Hkv, cap, d, n_past, n_new):
    import torch
    import compressive_memory_transformers_segment_amd as ia
    q, kc, vc, beta, M, z = _inputs(seed, dtype, B, Hq, Hkv, cap, d, n_past, n_new)
    h = ia.handle_for(q, kc, 1e-6, seq_len=cap)
    ref = torch.full_like(q, float("nan"))
    got = torch.full_like(q, float("nan"))
    assert _call("infini_attn_decode", h, q, kc, vc, n_past, beta, M, z, ref) == 0
    assert _call("infini_attn_decode_noalloc", h, q, kc, vc, n_past, beta, M, z, got) == 0
    torch.cuda.synchronize()
    return to_host64(got, dtype), to_host64(ref, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_decode_matches_decode_twice(dtype):
    # First call: the Llama-3-8B attention shape, 5 new rows near the end of a
    # 2048-row segment (2.7 MB of partials); second call: a smaller input.
    for (B, Hq, Hkv, cap, d, n_past, n_new) in [(1, 32, 8, 2048, 128, 2000, 5),
                                                (2, 4, 2, 300, 64, 37, 1)]:
        log(f"noalloc {dtype} B={B} Hq={Hq} Hkv={Hkv} cap={cap} d={d} n_past={n_past} "
            f"n_new={n_new}")
        got, ref = _both(7 + n_new, dtype, B, Hq, Hkv, cap, d, n_past, n_new)
        assert np.all(np.isfinite(ref))
        assert np.array_equal(got, ref), f"max diff {np.max(np.abs(got - ref))}"
        check(f"noalloc {dtype} n_new={n_new}", got, ref, "f32")


def test_noalloc_decode_rejects_requests_beyond_its_scratch():
    import torch
    import compressive_memory_transformers_segment_amd as ia
    from compressive_memory_transformers_segment_amd import _lib
    # 16 new rows of 32 heads against 2048 cached rows: 4 * 130 * 32 * 16 * 33
    # bytes (32 key splits and the retrieval slot) = 8.8 MB fits; 40 rows
    # (22 MB) do not.
    B, Hq, Hkv, cap, d = 1, 32, 8, 2048, 128
    for n_new, fits in ((16, True), (40, False)):
        need = 4 * (d + 2) * B * Hq * n_new * (-(-(cap - n_new + n_new) // 64) + 1)
        assert (need <= _lib.DECODE_SCRATCH_BYTES) == fits
        q, kc, vc, beta, M, z = _inputs(3, "bf16", B, Hq, Hkv, cap, d, cap - n_new, n_new)
        h = ia.handle_for(q, kc, 1e-6, seq_len=cap)
        out = torch.zeros_like(q)
        st = _call("infini_attn_decode_noalloc", h, q, kc, vc, cap - n_new, beta, M, z, out)
        torch.cuda.synchronize()
        if fits:
            assert st == 0
            assert bool(torch.isfinite(out.float()).all())
        else:
            assert st == _lib.ERR_SCRATCH
            assert int(torch.count_nonzero(out)) == 0  # nothing was enqueued
