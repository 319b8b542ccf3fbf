"""Plain fp64 definition of the Infini-attention forward pass (test infrastructure).

Only the test suite, ``__graft_entry__.smoke`` and ``bench.py``'s CPU baseline
may use this module. Every function works on float64 numpy arrays that the
caller has upcast exactly from the stored (fp32 or bf16) inputs.

Notation (per head):
    N        segment length; the input is cut into rows [s*N, min((s+1)*N, L)).
    sigma    ELU + 1 feature map.
    M, z     compressive memory (d_k x d_v) and its normaliser (d_k).
    beta     one learned gate scalar per query head; gamma = sigmoid(beta).

Readings taken where the pages leave a step open (each one is listed with its
reason in the design notes):
    * eps is added to the retrieval denominator only (1e-6 by default) and the
      same expression is used for the delta rule's inner retrieval.
    * ELU uses alpha = 1, so sigma(x) = x + 1 for x > 0 and exp(x) otherwise.
    * The dot-product scale 1/sqrt(d_k) applies inside the softmax only;
      sigma sees the unscaled q and k.
    * The causal mask is j <= i inside the current segment (diagonal kept).
    * gamma multiplies the memory branch; one beta per query head.
    * Grouped heads: query head h reads kv head h // (Hq / Hkv).
    * The last segment is shorter when L is not a multiple of N.
"""

from __future__ import annotations

import math
from typing import List, Optional, Tuple

import numpy as np

LINEAR = "linear"
DELTA = "delta"


def elu_plus_one(x: np.ndarray) -> np.ndarray:
    """sigma(x) = ELU(x) + 1 with alpha = 1: x + 1 for x > 0, exp(x) for x <= 0.

    [HF-repro] "Infini-Attention メカニズム", step Memory Retrieval (ELU + 1);
    [LNCB-review] "メモリの読み出し" (ELU+1 feature map).
    """
    x = np.asarray(x, dtype=np.float64)
    return np.where(x > 0.0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def gate_value(beta: np.ndarray) -> np.ndarray:
    """gamma = sigmoid(beta) = 1 / (1 + exp(-beta)), exact at beta = +-inf.

    [HF-repro] "Infini-Attention メカニズム", step Integration (a learned scalar
    beta through a sigmoid balances A_mem and A_dot); [LNCB-review]
    "長期情報と短期情報の統合" (per-head gate).
    """
    b = np.asarray(beta, dtype=np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-b))


def kv_head_of(h: int, n_q_heads: int, n_kv_heads: int) -> int:
    """Key/value head read by query head ``h`` (contiguous groups of Hq/Hkv)."""
    return h // (n_q_heads // n_kv_heads)


def segment_bounds(L: int, N: int) -> List[Tuple[int, int]]:
    """Row ranges of the fixed-length segments, the last one possibly shorter.

    [HF-repro] "Infini-Attention メカニズム", step Segmentation;
    [LNCB-review] "実装上の流れ" (split inside each layer's block).
    """
    if N < 1:
        raise ValueError("segment length must be >= 1")
    return [(s, min(s + N, L)) for s in range(0, L, N)]


def local_causal_attention(qs: np.ndarray, ks: np.ndarray, vs: np.ndarray) -> np.ndarray:
    """A_dot = softmax(mask(Q K^T / sqrt(d_k))) V inside one segment.

    Row i attends to rows j <= i of the same segment only.
    [HF-repro] "Infini-Attention メカニズム", step Local Attention (standard causal
    dot-product attention inside the current segment); [LNCB-review]
    "基本アイデア" (scaled dot-product attention per segment).
    """
    n, dk = qs.shape
    scores = (qs @ ks.T) / math.sqrt(dk)
    future = np.triu(np.ones((n, n), dtype=bool), k=1)
    scores = np.where(future, -np.inf, scores)
    scores = scores - scores.max(axis=1, keepdims=True)
    p = np.exp(scores)
    p = p / p.sum(axis=1, keepdims=True)
    return p @ vs


def local_causal_attention_rows(q_rows: np.ndarray, pos: np.ndarray, ks: np.ndarray,
                                vs: np.ndarray) -> np.ndarray:
    """A_dot for selected rows only: row r (at position pos[r] in its segment)
    attends to ks[:pos[r]+1], vs[:pos[r]+1]. Same definition as
    ``local_causal_attention``, evaluated one row at a time."""
    dk = q_rows.shape[1]
    out = np.empty((q_rows.shape[0], vs.shape[1]), dtype=np.float64)
    for r in range(q_rows.shape[0]):
        p_end = int(pos[r]) + 1
        sc = (ks[:p_end] @ q_rows[r]) / math.sqrt(dk)
        sc = sc - sc.max()
        w = np.exp(sc)
        out[r] = (w / w.sum()) @ vs[:p_end]
    return out


def memory_retrieval(qs: np.ndarray, M: np.ndarray, z: np.ndarray, eps: float) -> np.ndarray:
    """A_mem = sigma(Q) M_{s-1} / (sigma(Q) z_{s-1} + eps), row by row.

    [HF-repro] "Infini-Attention メカニズム", step Memory Retrieval (query through
    ELU+1 against M_{s-1}); [LNCB-review] "メモリの読み出し" (normalised by the
    running sum of past keys).
    """
    sq = elu_plus_one(qs)
    num = sq @ M
    den = sq @ z + eps
    return num / den[:, None]


def memory_update(ks: np.ndarray, vs: np.ndarray, M: np.ndarray, z: np.ndarray, mode: str,
                  eps: float) -> Tuple[np.ndarray, np.ndarray]:
    """One segment's write into (M, z); returns the new pair, inputs untouched.

    linear: M += sigma(K)^T V.
    delta:  M += sigma(K)^T (V - sigma(K) M / (sigma(K) z + eps)), i.e. only what
            the memory does not already return for these keys is written.
    both:   z += sum over the segment's rows of sigma(k).

    [HF-repro] "Infini-Attention メカニズム", step Memory Update (the segment's
    key/value states are added to the buffer); [LNCB-review] "メモリの更新"
    (outer-product accumulation, and the delta rule that writes only the
    difference); [aivaro-QA] section 4 (sigma(K)^T V accumulated into memory).
    """
    sk = elu_plus_one(ks)
    if mode == LINEAR:
        write = vs
    elif mode == DELTA:
        retrieved = (sk @ M) / (sk @ z + eps)[:, None]
        write = vs - retrieved
    else:
        raise ValueError(f"unknown update mode {mode!r}")
    return M + sk.T @ write, z + sk.sum(axis=0)


def infini_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, beta: np.ndarray,
                     M0: np.ndarray, z0: np.ndarray, seg_len: int, mode: str,
                     eps: float = 1e-6) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Full forward pass over all segments.

    q: [B, Hq, L, d_k]; k: [B, Hkv, L, d_k]; v: [B, Hkv, L, d_v]; beta: [Hq];
    M0: [B, Hkv, d_k, d_v]; z0: [B, Hkv, d_k]. Returns (out [B, Hq, L, d_v], M_S, z_S).

    Per segment: every query head computes its local attention and its
    retrieval from the state *before* this segment's update, mixes them with
    gamma = sigmoid(beta_h), then every kv head writes the segment into (M, z).
    Only (M, z) crosses segment boundaries.
    [HF-repro] "Infini-Attention メカニズム" (all six steps, in that order);
    [LNCB-review] "実装上の流れ" (local attention and retrieval, gate, then update
    with the current K/V and hand the memory on).
    """
    B, Hq, L, dk = q.shape
    Hkv = k.shape[1]
    dv = v.shape[3]
    if Hq % Hkv != 0:
        raise ValueError("query heads must be a multiple of kv heads")
    gamma = gate_value(beta)
    M = np.array(M0, dtype=np.float64, copy=True)
    z = np.array(z0, dtype=np.float64, copy=True)
    out = np.empty((B, Hq, L, dv), dtype=np.float64)
    for (a, e) in segment_bounds(L, seg_len):
        for b in range(B):
            for h in range(Hq):
                j = kv_head_of(h, Hq, Hkv)
                a_dot = local_causal_attention(q[b, h, a:e], k[b, j, a:e], v[b, j, a:e])
                a_mem = memory_retrieval(q[b, h, a:e], M[b, j], z[b, j], eps)
                out[b, h, a:e] = gamma[h] * a_mem + (1.0 - gamma[h]) * a_dot
        for b in range(B):
            for j in range(Hkv):
                M[b, j], z[b, j] = memory_update(k[b, j, a:e], v[b, j, a:e], M[b, j], z[b, j],
                                                 mode, eps)
    return out, M, z


def memory_chain(k: np.ndarray, v: np.ndarray, M0: np.ndarray, z0: np.ndarray, seg_len: int,
                 mode: str, eps: float = 1e-6, keep_states: bool = False,
                 upcast=None) -> Tuple[np.ndarray, np.ndarray, Optional[list]]:
    """The (M, z) recurrence alone for one head: k [L, d_k], v [L, d_v].

    Returns (M_S, z_S, states) where ``states`` (when kept) lists the state
    *before* each segment, i.e. what that segment's retrieval reads.
    ``upcast`` (optional) maps a stored slice to fp64 so a large stored tensor
    can be streamed one segment at a time.
    [HF-repro] "Infini-Attention メカニズム", steps Memory Update and State Transfer.
    """
    M = np.array(M0, dtype=np.float64, copy=True)
    z = np.array(z0, dtype=np.float64, copy=True)
    states = [] if keep_states else None
    L = k.shape[0]
    for (a, e) in segment_bounds(L, seg_len):
        if keep_states:
            states.append((M.copy(), z.copy()))
        ks = k[a:e] if upcast is None else upcast(k[a:e])
        vs = v[a:e] if upcast is None else upcast(v[a:e])
        M, z = memory_update(ks, vs, M, z, mode, eps)
    return M, z, states


def streaming_decode(q: np.ndarray, k: np.ndarray, v: np.ndarray, beta: np.ndarray,
                     M0: np.ndarray, z0: np.ndarray, seg_len: int, mode: str, chunk: int = 1,
                     eps: float = 1e-6) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Streaming inference: the tokens arrive in chunks of ``chunk`` rows (a
    chunk never crosses a segment boundary), and only the current segment's
    K/V rows plus (M, z) are kept.

    For each arriving row at position p of its segment: local causal attention
    over the cached rows 0..p of the segment, retrieval from the state before
    the segment, the gate mix. When the segment's last row has arrived (or the
    stream ends inside a segment), the cached rows are written into (M, z) and
    the cache is emptied. Same shapes and return values as ``infini_attention``.

    [HF-repro] "Infini-Attention メカニズム", steps Memory Update and State
    Transfer (only the memory is handed on, the past segment's K/V is not
    kept); [LNCB-review] "実装上の流れ" (attend and retrieve, then update the
    memory with the current K/V and move to the next segment).
    """
    B, Hq, L, dk = q.shape
    Hkv = k.shape[1]
    dv = v.shape[3]
    if chunk < 1:
        raise ValueError("chunk must be >= 1")
    gamma = gate_value(beta)
    M = np.array(M0, dtype=np.float64, copy=True)
    z = np.array(z0, dtype=np.float64, copy=True)
    out = np.empty((B, Hq, L, dv), dtype=np.float64)
    cache_k = np.zeros((B, Hkv, seg_len, dk), dtype=np.float64)
    cache_v = np.zeros((B, Hkv, seg_len, dv), dtype=np.float64)
    n_cached = 0
    t = 0
    while t < L:
        n_new = min(chunk, seg_len - n_cached, L - t)
        # the new rows join the cache before they attend (each sees itself)
        cache_k[:, :, n_cached:n_cached + n_new] = k[:, :, t:t + n_new]
        cache_v[:, :, n_cached:n_cached + n_new] = v[:, :, t:t + n_new]
        pos = np.arange(n_cached, n_cached + n_new)
        for b in range(B):
            for h in range(Hq):
                j = kv_head_of(h, Hq, Hkv)
                rows = q[b, h, t:t + n_new]
                a_dot = local_causal_attention_rows(rows, pos, cache_k[b, j], cache_v[b, j])
                a_mem = memory_retrieval(rows, M[b, j], z[b, j], eps)
                out[b, h, t:t + n_new] = gamma[h] * a_mem + (1.0 - gamma[h]) * a_dot
        n_cached += n_new
        t += n_new
        if n_cached == seg_len or t == L:
            for b in range(B):
                for j in range(Hkv):
                    M[b, j], z[b, j] = memory_update(cache_k[b, j, :n_cached],
                                                     cache_v[b, j, :n_cached], M[b, j], z[b, j],
                                                     mode, eps)
            n_cached = 0
    return out, M, z


def infini_block(x: np.ndarray, wq: np.ndarray, wk: np.ndarray, wv: np.ndarray, wo: np.ndarray,
                 beta: np.ndarray, M0: np.ndarray, z0: np.ndarray, seg_len: int, mode: str,
                 n_q_heads: int, n_kv_heads: int,
                 eps: float = 1e-6) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """The layer around the mechanism: query, key and value states are linear
    projections of the layer input x [B, L, d_model] (head h takes columns
    h*d .. h*d + d - 1 of x @ W), the Infini-attention forward runs on them,
    and the heads of each row, side by side, go through the output projection.
    Returns (y [B, L, d_model], M_S, z_S).

    [HF-repro] "Infini-Attention メカニズム" (the mechanism consumes the
    layer's own query / key / value states); [LNCB-review] "基本アイデア" (it
    takes the place of the attention inside each layer's block).
    """
    B, L, dm = x.shape
    d = wq.shape[1] // n_q_heads

    def heads(w, n):
        return (x @ w).reshape(B, L, n, d).transpose(0, 2, 1, 3)

    q, k, v = heads(wq, n_q_heads), heads(wk, n_kv_heads), heads(wv, n_kv_heads)
    out, M, z = infini_attention(q, k, v, beta, M0, z0, seg_len, mode, eps)
    y = out.transpose(0, 2, 1, 3).reshape(B, L, n_q_heads * d) @ wo
    return y, M, z


def _elu_plus_one_grad(x: np.ndarray) -> np.ndarray:
    """d sigma / dx: 1 for x > 0, exp(x) otherwise."""
    return np.where(x > 0.0, 1.0, np.exp(np.minimum(x, 0.0)))


def infini_attention_backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, beta: np.ndarray,
                              M0: np.ndarray, z0: np.ndarray, seg_len: int, mode: str,
                              d_out: np.ndarray, d_M: Optional[np.ndarray] = None,
                              d_z: Optional[np.ndarray] = None, eps: float = 1e-6):
    """Gradients of L = <d_out, out> + <d_M, M_S> + <d_z, z_S> with respect to
    (q, k, v, beta, M0, z0), for the forward pass of ``infini_attention``.

    Backpropagation through time over the segments (the training setting of
    [LNCB-review] "実装上の流れ" and of [HF-repro]'s reproduction, where the
    memory carries gradient from later segments to earlier ones): the segments
    are visited in reverse, carrying the gradient of the state after each one.
    Per segment, in reverse order of the forward's steps:
      gate:       d gamma = sum d_out (A_mem - A_dot), d beta = d gamma g (1 - g);
      attention:  softmax backward of A_dot = P V with d A_dot = (1 - g) d_out;
      retrieval:  A_mem = n / den with n = sigma(Q) M_{s-1}, den = sigma(Q) z_{s-1}
                  + eps: d n = d A_mem / den, d den = -sum(d A_mem n) / den^2;
      update:     the linear or delta write of (K_s, V_s) into (M, z), whose
                  gradient flows into K_s, V_s and the earlier state.
    Returns (dq, dk, dv, dbeta, dM0, dz0).
    """
    B, Hq, L, dk_ = q.shape
    Hkv = k.shape[1]
    dv_ = v.shape[3]
    grp = Hq // Hkv
    gamma = gate_value(beta)
    gsl = gamma * (1.0 - gamma)  # d gamma / d beta (0 at the infinities)
    dq = np.zeros_like(q, dtype=np.float64)
    dk = np.zeros_like(k, dtype=np.float64)
    dv = np.zeros_like(v, dtype=np.float64)
    dbeta = np.zeros(Hq, dtype=np.float64)
    dM0 = np.zeros((B, Hkv, dk_, dv_)) if d_M is None else np.array(d_M, dtype=np.float64)
    dz0 = np.zeros((B, Hkv, dk_)) if d_z is None else np.array(d_z, dtype=np.float64)
    bounds = segment_bounds(L, seg_len)
    scale = 1.0 / math.sqrt(dk_)
    for b in range(B):
        for j in range(Hkv):
            _, _, states = memory_chain(k[b, j], v[b, j], M0[b, j], z0[b, j], seg_len, mode, eps,
                                        keep_states=True)
            gM, gz = dM0[b, j], dz0[b, j]  # gradient of the state after the segment
            for s in reversed(range(len(bounds))):
                a, e = bounds[s]
                Mp, zp = states[s]
                ks, vs = k[b, j, a:e], v[b, j, a:e]
                n = e - a
                gMp, gzp = gM.copy(), gz.copy()  # the state passes through the update
                for h in range(j * grp, (j + 1) * grp):
                    Q = q[b, h, a:e]
                    dO = d_out[b, h, a:e]
                    # forward values of this segment
                    S = (Q @ ks.T) * scale
                    S = np.where(np.triu(np.ones((n, n), dtype=bool), k=1), -np.inf, S)
                    P = np.exp(S - S.max(axis=1, keepdims=True))
                    P = P / P.sum(axis=1, keepdims=True)
                    a_dot = P @ vs
                    sq = elu_plus_one(Q)
                    num = sq @ Mp
                    den = sq @ zp + eps
                    a_mem = num / den[:, None]
                    # gate
                    dbeta[h] += np.sum(dO * (a_mem - a_dot)) * gsl[h]
                    # local attention
                    dA = (1.0 - gamma[h]) * dO
                    dv[b, j, a:e] += P.T @ dA
                    dP = dA @ vs.T
                    dS = P * (dP - np.sum(dP * P, axis=1, keepdims=True))
                    dq[b, h, a:e] += (dS @ ks) * scale
                    dk[b, j, a:e] += (dS.T @ Q) * scale
                    # retrieval
                    dAm = gamma[h] * dO
                    dnum = dAm / den[:, None]
                    dden = -np.sum(dAm * num, axis=1) / den ** 2
                    dsq = dnum @ Mp.T + dden[:, None] * zp[None, :]
                    gMp += sq.T @ dnum
                    gzp += sq.T @ dden
                    dq[b, h, a:e] += dsq * _elu_plus_one_grad(Q)
                # memory update of this segment
                sk = elu_plus_one(ks)
                if mode == LINEAR:
                    write = vs
                    dsk = write @ gM.T + gz[None, :]
                    dv[b, j, a:e] += sk @ gM
                elif mode == DELTA:
                    numk = sk @ Mp
                    denk = sk @ zp + eps
                    write = vs - numk / denk[:, None]
                    dsk = write @ gM.T + gz[None, :]
                    dW = sk @ gM
                    dv[b, j, a:e] += dW
                    dR = -dW
                    dnumk = dR / denk[:, None]
                    ddenk = -np.sum(dR * numk, axis=1) / denk ** 2
                    dsk += dnumk @ Mp.T + ddenk[:, None] * zp[None, :]
                    gMp += sk.T @ dnumk
                    gzp += sk.T @ ddenk
                else:
                    raise ValueError(f"unknown update mode {mode!r}")
                dk[b, j, a:e] += dsk * _elu_plus_one_grad(ks)
                gM, gz = gMp, gzp
            dM0[b, j], dz0[b, j] = gM, gz
    return dq, dk, dv, dbeta, dM0, dz0
