"""What a NaN input produces on the GPU paths, against the oracle: a NaN in q
or k gives exactly the oracle's NaN pattern in out, M and z (its own row; or
the rows at or after it in its segment, every later segment of its kv group
and the state), with the finite elements within the usual tolerance. A NaN in
one column of v gives NaN in that column for the rows at or after it, the
later segments and M, and may also reach the rows before it that share its
64-key tile: the kernels multiply it by their exact-zero masked probabilities.
The bf16 fused kernel runs with the IEEE mode bit off, so its row maxima skip
NaN scores; the NaN still reaches the row through its exponentials."""

import numpy as np
import pytest

import synth
from parity import check, log, run_gpu, run_oracle

pytestmark = pytest.mark.gpu

L, N, D = 300, 128, 64  # segments of 128, 128, 44 rows


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import compressive_memory_transformers_segment_amd as ia
    ia.load()
    yield
    ia.release_handles()


def _case(dtype, seed):
    return synth.random_case(seed, B=1, Hq=4, Hkv=2, L=L, dk=D, dv=D, dtype=dtype,
                             nonzero_state=True, scale=1.5 / np.sqrt(D) * 4)


def _nan_bits(dtype):
    return np.uint16(0x7FC0) if dtype == "bf16" else np.float32("nan")


def _finite_close(tag, gpu, ref, dtype):
    for name, g, o, st in zip(("out", "M", "z"), gpu, ref, (False, True, True)):
        fin = np.isfinite(o) & np.isfinite(g)
        if fin.any():
            check(f"{tag} {name} (finite part)", g[fin], o[fin], dtype, state=st)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mode", ["linear", "delta"])
@pytest.mark.parametrize("which", ["q", "k"])
def test_nan_in_q_or_k_matches_the_oracle(dtype, mode, which):
    inp = _case(dtype, 71)
    if which == "q":
        inp["q"][0, 1, 150, 2] = _nan_bits(dtype)
    else:
        inp["k"][0, 0, 170, 7] = _nan_bits(dtype)
    tag = f"nan in {which} {dtype} {mode}"
    log(tag)
    gpu = run_gpu(inp, dtype, N, mode)
    with np.errstate(invalid="ignore"):
        ref = run_oracle(inp, dtype, N, mode)
    for name, g, o in zip(("out", "M", "z"), gpu, ref):
        assert np.array_equal(np.isnan(g), np.isnan(o)), (
            f"{tag} {name}: NaN pattern differs ({int(np.isnan(g).sum())} vs "
            f"{int(np.isnan(o).sum())} NaN elements)")
        assert not np.any(np.isinf(g)), f"{tag} {name}: infinite values"
    _finite_close(tag, gpu, ref, dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mode", ["linear", "delta"])
def test_nan_in_v_reaches_its_column(dtype, mode):
    inp = _case(dtype, 72)
    t, col = 140, 9  # segment 1 (rows 128..255), kv head 1 (query heads 2, 3)
    inp["v"][0, 1, t, col] = _nan_bits(dtype)
    tag = f"nan in v {dtype} {mode}"
    log(tag)
    out, M, z = run_gpu(inp, dtype, N, mode)
    with np.errstate(invalid="ignore"):
        ref = run_oracle(inp, dtype, N, mode)
    must = np.zeros(out.shape, bool)
    must[0, 2:, t:, col] = True              # rows >= t and every later segment
    may = must.copy()
    tile0 = N + (t - N) // 64 * 64            # first row of the key tile holding t
    may[0, 2:, tile0:t, col] = True          # earlier rows of that tile
    got = np.isnan(out)
    assert np.all(got[must]), f"{tag}: a dependent element is not NaN"
    assert not np.any(got & ~may), f"{tag}: NaN outside its column's reach"
    assert np.all(np.isnan(M[0, 1, :, col]))
    assert np.all(np.isfinite(np.delete(M[0, 1], col, axis=1))) and np.all(np.isfinite(M[0, 0]))
    assert np.all(np.isfinite(z))
    # (the oracle's own matrix product may also spread the NaN to earlier rows
    # of the segment through its exact zeros; those elements are not compared)
    fin = ~may & np.isfinite(ref[0])
    check(f"{tag} out (outside the column's reach)", out[fin], ref[0][fin], dtype)
