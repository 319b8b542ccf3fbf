"""Independent references used to pin the fp64 oracle.

None of these share code with the oracle: each one evaluates the method by a
different route (scalar loops, exact rationals, a dense masked matrix with no
recurrence, a library attention routine), so a dropped term, a wrong sign or
index, or a transposed operand in the oracle shows up as a mismatch.
"""

from __future__ import annotations

import math
from fractions import Fraction
from typing import List

import numpy as np


# ----------------------------------------------------------------------------
# P-7: token-by-token scalar brute force (pure Python, tiny inputs only)
# ----------------------------------------------------------------------------

def _sig(x: float) -> float:
    return x + 1.0 if x > 0.0 else math.exp(x)


def brute_force(q, k, v, beta, M0, z0, N: int, mode: str, eps: float):
    """Every output element as an explicit sum; every memory write as explicit
    per-token outer products. Inputs are nested lists / arrays of floats."""
    q = np.asarray(q, dtype=np.float64).tolist()
    k = np.asarray(k, dtype=np.float64).tolist()
    v = np.asarray(v, dtype=np.float64).tolist()
    B, Hq, L, dk = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Hkv = len(k[0])
    dv = len(v[0][0][0])
    grp = Hq // Hkv
    Ms = [[[list(map(float, row)) for row in np.asarray(M0)[b, j]] for j in range(Hkv)]
          for b in range(B)]
    zs = [[list(map(float, np.asarray(z0)[b, j])) for j in range(Hkv)] for b in range(B)]
    out = [[[[0.0] * dv for _ in range(L)] for _ in range(Hq)] for _ in range(B)]
    starts = list(range(0, L, N))
    for a in starts:
        e = min(a + N, L)
        for b in range(B):
            for h in range(Hq):
                j = h // grp
                g = 1.0 / (1.0 + math.exp(-float(beta[h]))) if math.isfinite(beta[h]) else (
                    1.0 if beta[h] > 0 else 0.0)
                for i in range(a, e):
                    # local causal softmax attention over rows a..i
                    sc = []
                    for t in range(a, i + 1):
                        dot = 0.0
                        for c in range(dk):
                            dot += q[b][h][i][c] * k[b][j][t][c]
                        sc.append(dot / math.sqrt(dk))
                    mx = max(sc)
                    w = [math.exp(s - mx) for s in sc]
                    tot = sum(w)
                    # retrieval from the state before this segment
                    sq = [_sig(q[b][h][i][c]) for c in range(dk)]
                    den = eps
                    for c in range(dk):
                        den += sq[c] * zs[b][j][c]
                    for col in range(dv):
                        adot = 0.0
                        for t in range(a, i + 1):
                            adot += w[t - a] * v[b][j][t][col]
                        adot /= tot
                        num = 0.0
                        for c in range(dk):
                            num += sq[c] * Ms[b][j][c][col]
                        out[b][h][i][col] = g * (num / den) + (1.0 - g) * adot
        # memory writes, token by token, all reading the segment-start state
        for b in range(B):
            for j in range(Hkv):
                M_old = [row[:] for row in Ms[b][j]]
                z_old = zs[b][j][:]
                for t in range(a, e):
                    sk = [_sig(k[b][j][t][c]) for c in range(dk)]
                    if mode == "delta":
                        den = eps
                        for c in range(dk):
                            den += sk[c] * z_old[c]
                        wv = []
                        for col in range(dv):
                            r = 0.0
                            for c in range(dk):
                                r += sk[c] * M_old[c][col]
                            wv.append(v[b][j][t][col] - r / den)
                    else:
                        wv = [v[b][j][t][col] for col in range(dv)]
                    for c in range(dk):
                        for col in range(dv):
                            Ms[b][j][c][col] += sk[c] * wv[col]
                        zs[b][j][c] += sk[c]
    return np.array(out), np.array(Ms), np.array(zs)


# ----------------------------------------------------------------------------
# P-6: exact rational evaluation when every q, k entry is positive
# ----------------------------------------------------------------------------

def exact_memory_branch(q, k, v, M0, z0, N: int, mode: str, eps: float):
    """A_mem, M and z in exact rational arithmetic.

    Requires all q, k > 0 so that ELU+1 is the rational map x -> x + 1.
    Inputs are floats (converted exactly with ``Fraction``); returns nested
    Fraction lists (out, M, z). Single (b, head) slice: q [L, dk], k [L, dk],
    v [L, dv], M0 [dk, dv], z0 [dk].
    """
    F = Fraction
    qf = [[F(float(x)) for x in row] for row in np.asarray(q)]
    kf = [[F(float(x)) for x in row] for row in np.asarray(k)]
    vf = [[F(float(x)) for x in row] for row in np.asarray(v)]
    M = [[F(float(x)) for x in row] for row in np.asarray(M0)]
    z = [F(float(x)) for x in np.asarray(z0)]
    e = F(float(eps))
    L, dk, dv = len(qf), len(qf[0]), len(vf[0])
    assert all(x > 0 for row in qf for x in row) and all(x > 0 for row in kf for x in row)
    out: List[List[Fraction]] = []
    for a in range(0, L, N):
        stop = min(a + N, L)
        for i in range(a, stop):
            sq = [x + 1 for x in qf[i]]
            den = sum((sq[c] * z[c] for c in range(dk)), F(0)) + e
            out.append([sum((sq[c] * M[c][col] for c in range(dk)), F(0)) / den
                        for col in range(dv)])
        newM = [row[:] for row in M]
        newz = z[:]
        for t in range(a, stop):
            sk = [x + 1 for x in kf[t]]
            if mode == "delta":
                den = sum((sk[c] * z[c] for c in range(dk)), F(0)) + e
                wv = [vf[t][col] - sum((sk[c] * M[c][col] for c in range(dk)), F(0)) / den
                      for col in range(dv)]
            else:
                wv = vf[t]
            for c in range(dk):
                for col in range(dv):
                    newM[c][col] += sk[c] * wv[col]
                newz[c] += sk[c]
        M, z = newM, newz
    return out, M, z


# ----------------------------------------------------------------------------
# P-2: dense block-causal normalised linear attention (no recurrence)
# ----------------------------------------------------------------------------

def dense_block_causal_linear(q, k, v, M0, z0, N: int, eps: float):
    """A_mem for one (b, head) slice under the linear rule, from an L x L matrix.

    A_mem[i] = (sig(q_i) M0 + sum_{j < start(i)} (sig(q_i).sig(k_j)) v_j)
             / (sig(q_i).z0 + sum_{j < start(i)} sig(q_i).sig(k_j) + eps)
    where start(i) is the first row of i's segment.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    L = q.shape[0]
    fq = np.where(q > 0, q + 1.0, np.exp(np.minimum(q, 0.0)))
    fk = np.where(k > 0, k + 1.0, np.exp(np.minimum(k, 0.0)))
    seg = np.arange(L) // N
    past = seg[None, :] < seg[:, None]  # key j lies in an earlier segment than query i
    W = (fq @ fk.T) * past
    num = fq @ np.asarray(M0, dtype=np.float64) + W @ v
    den = fq @ np.asarray(z0, dtype=np.float64) + W.sum(axis=1) + eps
    return num / den[:, None]


# ----------------------------------------------------------------------------
# P-1: library attention per segment
# ----------------------------------------------------------------------------

def sdpa_per_segment(q, k, v, N: int):
    """torch's scaled_dot_product_attention (causal) in fp64 on the CPU, applied
    segment by segment; q [B, Hq, L, dk], k/v [B, Hkv, L, d] with kv heads
    repeated to match the query heads."""
    import torch
    import torch.nn.functional as Fn

    qt = torch.from_numpy(np.asarray(q, dtype=np.float64))
    kt = torch.from_numpy(np.asarray(k, dtype=np.float64))
    vt = torch.from_numpy(np.asarray(v, dtype=np.float64))
    g = qt.shape[1] // kt.shape[1]
    kt = kt.repeat_interleave(g, dim=1)
    vt = vt.repeat_interleave(g, dim=1)
    L = qt.shape[2]
    outs = []
    for a in range(0, L, N):
        e = min(a + N, L)
        outs.append(Fn.scaled_dot_product_attention(qt[:, :, a:e], kt[:, :, a:e], vt[:, :, a:e],
                                                    is_causal=True))
    return torch.cat(outs, dim=2).numpy()
