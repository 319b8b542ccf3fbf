"""What a NaN input produces, on the oracle (CPU): NaN reaches every output
element that depends on the NaN element in exact arithmetic, and nothing that
does not. A NaN in q reaches its own output row; a NaN in k reaches the rows
at or after it in its segment (every query head of its group), every later
segment of the group through the memory, and the state; a NaN in one column
of v reaches that column. (Rows before a NaN value in its segment multiply it
by an exact zero probability; whether that yields NaN depends on how the
product is evaluated, so those elements are left unchecked.)"""

import numpy as np
import pytest

import oracle

B, HQ, HKV, L, N, D = 1, 4, 2, 24, 8, 5  # three segments of 8


def _inputs(seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, HQ, L, D))
    k = rng.standard_normal((B, HKV, L, D))
    v = rng.standard_normal((B, HKV, L, D))
    beta = rng.standard_normal(HQ)
    M0 = 0.1 * rng.standard_normal((B, HKV, D, D))
    z0 = rng.uniform(0.5, 2.0, (B, HKV, D))
    return q, k, v, beta, M0, z0


def _run(q, k, v, beta, M0, z0, mode):
    with np.errstate(invalid="ignore"):
        return oracle.infini_attention(q, k, v, beta, M0, z0, N, mode, 1e-6)


@pytest.mark.parametrize("mode", ["linear", "delta"])
def test_nan_in_q_reaches_only_its_row(mode):
    q, k, v, beta, M0, z0 = _inputs(1)
    q[0, 1, 10, 2] = np.nan
    out, M, z = _run(q, k, v, beta, M0, z0, mode)
    assert np.all(np.isnan(out[0, 1, 10]))
    mask = np.ones(out.shape, bool)
    mask[0, 1, 10] = False
    assert np.all(np.isfinite(out[mask])) and np.all(np.isfinite(M)) and np.all(np.isfinite(z))


@pytest.mark.parametrize("mode", ["linear", "delta"])
def test_nan_in_k_reaches_later_rows_segments_and_state(mode):
    q, k, v, beta, M0, z0 = _inputs(2)
    t, c = 11, 3  # segment 1 (rows 8..15), kv head 0 (query heads 0 and 1)
    k[0, 0, t, c] = np.nan
    out, M, z = _run(q, k, v, beta, M0, z0, mode)
    assert np.all(np.isnan(out[0, :2, t:]))             # rows >= t and later segments
    assert np.all(np.isfinite(out[0, :2, :t]))          # earlier rows never see it
    assert np.all(np.isfinite(out[0, 2:]))              # other kv group
    assert np.isnan(z[0, 0, c]) and np.all(np.isfinite(np.delete(z[0, 0], c)))
    assert np.all(np.isfinite(z[0, 1])) and np.all(np.isfinite(M[0, 1]))
    if mode == "linear":  # only row c of M is written with sigma(k)_c
        assert np.all(np.isnan(M[0, 0, c])) and np.all(np.isfinite(np.delete(M[0, 0], c, axis=0)))
    else:  # the delta write divides by sigma(k).z, which is NaN: every entry
        assert np.all(np.isnan(M[0, 0]))


@pytest.mark.parametrize("mode", ["linear", "delta"])
def test_nan_in_v_reaches_its_column(mode):
    q, k, v, beta, M0, z0 = _inputs(3)
    t, col = 13, 4  # segment 1, kv head 1 (query heads 2 and 3)
    v[0, 1, t, col] = np.nan
    out, M, z = _run(q, k, v, beta, M0, z0, mode)
    assert np.all(np.isnan(out[0, 2:, t:, col]))        # rows >= t, later segments (memory)
    assert np.all(np.isfinite(np.delete(out[0, 2:], col, axis=2)))  # other columns
    assert np.all(np.isfinite(out[0, 2:, :N]))          # the segment before it
    assert np.all(np.isfinite(out[0, :2]))
    assert np.all(np.isnan(M[0, 1, :, col]))
    assert np.all(np.isfinite(np.delete(M[0, 1], col, axis=1))) and np.all(np.isfinite(M[0, 0]))
    assert np.all(np.isfinite(z))
