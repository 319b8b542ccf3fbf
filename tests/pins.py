"""Pins for the fp64 oracle: each function checks the oracle module ``ora``
against something other than itself (a library routine, a closed form, exact
rational arithmetic, a brute force, or an invariant the method fixes) and
raises AssertionError on a mismatch. They take the module as an argument so a
test can plant a mistake in it and show that some pin catches it.
"""

from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np

import independent as ind
from synth import as_f64, random_case

INF = float("inf")
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")


def case64(seed, B, Hq, Hkv, L, dk, dv, **kw):
    c = random_case(seed, B, Hq, Hkv, L, dk, dv, **kw)
    return dict(q=as_f64(c["q"], "f32"), k=as_f64(c["k"], "f32"), v=as_f64(c["v"], "f32"),
                beta=c["beta"].astype(np.float64), M0=c["M0"].astype(np.float64),
                z0=c["z0"].astype(np.float64), eps=1e-6)


def run(ora, c, N, mode, beta=None):
    b = c["beta"] if beta is None else np.asarray(beta, dtype=np.float64)
    return ora.infini_attention(c["q"], c["k"], c["v"], b, c["M0"], c["z0"], N, mode, c["eps"])


def close(a, b, rtol=1e-12, atol=1e-12, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert np.all(np.isfinite(a)) and np.all(np.isfinite(b)), f"{what}: non-finite values"
    err = np.max(np.abs(a - b) - rtol * np.abs(b)) if a.size else -1.0
    assert err <= atol, f"{what}: max excess error {err:.3e}"


# Shapes with a distinct size on every axis and a ragged last segment, so that a
# transposed axis or a wrong index cannot hide.
SHAPE = dict(B=2, Hq=6, Hkv=3, L=10, dk=3, dv=5)
N_RAGGED = 4  # segments of 4, 4, 2


def pin_sigma_library(ora):
    """sigma = ELU(alpha=1) + 1 (a library special case)."""
    import torch
    x = np.linspace(-6.0, 6.0, 1201)
    ref = torch.nn.functional.elu(torch.from_numpy(x), alpha=1.0).numpy() + 1.0
    close(ora.elu_plus_one(x), ref, rtol=1e-15, atol=1e-15, what="sigma")
    assert np.all(ora.elu_plus_one(x) > 0.0)


def pin_gate_library(ora):
    """gamma = sigmoid(beta), exact at the infinities."""
    import torch
    b = np.linspace(-30.0, 30.0, 601)
    close(ora.gate_value(b), torch.sigmoid(torch.from_numpy(b)).numpy(), rtol=1e-14, atol=1e-15,
          what="gate")
    g = ora.gate_value(np.array([-INF, INF]))
    assert g[0] == 0.0 and g[1] == 1.0


def pin_golden(ora):
    """Hand-derived closed forms (tests/golden/hand_cases.json)."""
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    env = {"__builtins__": {}, "exp": math.exp, "sqrt": math.sqrt}
    for cs in cases:
        eps = float(cs["eps"])
        beta = np.array([float(x) for x in cs["beta"]], dtype=np.float64)
        out, M, z = ora.infini_attention(np.array(cs["q"], dtype=np.float64),
                                         np.array(cs["k"], dtype=np.float64),
                                         np.array(cs["v"], dtype=np.float64), beta,
                                         np.array(cs["M0"], dtype=np.float64),
                                         np.array(cs["z0"], dtype=np.float64),
                                         int(cs["seg_len"]), cs["mode"], eps)
        ev = lambda t: np.vectorize(lambda s: float(eval(s, env, {"eps": eps})))(np.array(t))
        for name, got in (("out", out), ("M", M), ("z", z)):
            close(got, ev(cs["expected"][name]), rtol=1e-13, atol=1e-15,
                  what=f"golden {cs['name']} {name}")


def pin_p1_sdpa(ora):
    """beta = -inf gives gamma = 0: out must be per-segment causal SDPA."""
    for N, scale in ((N_RAGGED, 1.5), (3, None), (10, 2.0)):
        c = case64(11 + N, scale=scale, **SHAPE)
        out, _, _ = run(ora, c, N, "delta", beta=np.full(SHAPE["Hq"], -INF))
        close(out, ind.sdpa_per_segment(c["q"], c["k"], c["v"], N), rtol=1e-11, atol=1e-12,
              what=f"P-1 N={N}")


def pin_p2_dense_linear(ora):
    """beta = +inf gives out = A_mem; under the linear rule it must equal dense
    block-causal normalised linear attention (an L x L mask, no recurrence)."""
    for nz in (False, True):
        c = case64(21, scale=1.3, nonzero_state=nz, **SHAPE)
        out, _, _ = run(ora, c, N_RAGGED, "linear", beta=np.full(SHAPE["Hq"], INF))
        g = SHAPE["Hq"] // SHAPE["Hkv"]
        for b in range(SHAPE["B"]):
            for h in range(SHAPE["Hq"]):
                j = h // g
                ref = ind.dense_block_causal_linear(c["q"][b, h], c["k"][b, j], c["v"][b, j],
                                                    c["M0"][b, j], c["z0"][b, j], N_RAGGED,
                                                    c["eps"])
                close(out[b, h], ref, rtol=1e-10, atol=1e-12, what=f"P-2 b{b} h{h} nz={nz}")


def pin_p3_linear_closed_form(ora):
    """Linear rule: M_S = M0 + sum_t sig(k_t)^T v_t over all rows, z_S = z0 +
    sum_t sig(k_t); hence (M_S, z_S) does not depend on the segment length."""
    c = case64(31, nonzero_state=True, scale=1.2, **SHAPE)
    x = c["k"]
    sk = np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))
    M_ref = c["M0"] + np.einsum("bhld,bhle->bhde", sk, c["v"])
    z_ref = c["z0"] + sk.sum(axis=2)
    for N in (1, 3, N_RAGGED, SHAPE["L"], 64):
        _, M, z = run(ora, c, N, "linear")
        close(M, M_ref, rtol=1e-12, atol=1e-12, what=f"P-3 M N={N}")
        close(z, z_ref, rtol=1e-13, atol=1e-13, what=f"P-3 z N={N}")


def pin_p4_zero_start(ora):
    """M0 = 0, z0 = 0: the first segment's A_mem is exactly 0 (so beta = +inf
    gives exact zeros there), and the first delta write equals the linear one."""
    c = case64(41, scale=1.5, **SHAPE)
    out, _, _ = run(ora, c, N_RAGGED, "delta", beta=np.full(SHAPE["Hq"], INF))
    assert np.all(out[:, :, :N_RAGGED] == 0.0), "P-4: first segment A_mem not exactly 0"
    assert np.all(np.abs(out[:, :, N_RAGGED:]) > 0.0), "P-4: later segments must read memory"
    ks, vs = c["k"][0, 0, :N_RAGGED], c["v"][0, 0, :N_RAGGED]
    Z = np.zeros((SHAPE["dk"], SHAPE["dv"]))
    zz = np.zeros(SHAPE["dk"])
    Ml, zl = ora.memory_update(ks, vs, Z, zz, "linear", c["eps"])
    Md, zd = ora.memory_update(ks, vs, Z, zz, "delta", c["eps"])
    assert np.array_equal(Ml, Md) and np.array_equal(zl, zd), "P-4: first delta != linear write"


def pin_p5_delta_fixed_point(ora):
    """Writing exactly what the memory already returns for these keys leaves M
    unchanged (the delta rule writes only the difference); z still grows."""
    rng = np.random.default_rng(51)
    dk, dv, n = 4, 6, 7
    M = rng.standard_normal((dk, dv))
    z = np.abs(rng.standard_normal(dk)) * 3.0 + 0.5
    ks = rng.standard_normal((n, dk))
    sk = np.where(ks > 0, ks + 1.0, np.exp(np.minimum(ks, 0.0)))
    vs = (sk @ M) / (sk @ z + 1e-6)[:, None]
    M2, z2 = ora.memory_update(ks, vs, M, z, "delta", 1e-6)
    close(M2, M, rtol=1e-12, atol=1e-12, what="P-5 M unchanged")
    close(z2, z + sk.sum(axis=0), rtol=1e-14, atol=1e-14, what="P-5 z")
    # and a write that differs does change M (the pin is not vacuous)
    M3, _ = ora.memory_update(ks, vs + 1.0, M, z, "delta", 1e-6)
    assert np.max(np.abs(M3 - M)) > 1e-3


def pin_p6_exact(ora):
    """All q, k > 0 and dyadic: ELU+1 is x -> x+1, so with beta = +inf the whole
    memory branch is rational; compare with exact Fraction arithmetic."""
    rng = np.random.default_rng(61)
    B, Hq, Hkv, L, dk, dv, N = 1, 2, 1, 9, 3, 4, 4
    for mode in ("linear", "delta"):
        for nz in (False, True):
            q = rng.integers(1, 16, (B, Hq, L, dk)) / 8.0
            k = rng.integers(1, 16, (B, Hkv, L, dk)) / 8.0
            v = rng.integers(-16, 16, (B, Hkv, L, dv)) / 8.0
            M0 = (rng.integers(-8, 8, (B, Hkv, dk, dv)) / 4.0) if nz else np.zeros((B, Hkv, dk, dv))
            z0 = (rng.integers(1, 8, (B, Hkv, dk)) / 2.0) if nz else np.zeros((B, Hkv, dk))
            eps = 1e-6
            out, M, z = ora.infini_attention(q, k, v, np.full(Hq, INF), M0, z0, N, mode, eps)
            for h in range(Hq):
                eo, eM, ez = ind.exact_memory_branch(q[0, h], k[0, 0], v[0, 0], M0[0, 0], z0[0, 0],
                                                     N, mode, eps)
                close(out[0, h], np.array([[float(x) for x in r] for r in eo]), rtol=1e-12,
                      atol=1e-14, what=f"P-6 out {mode} nz={nz}")
            close(M[0, 0], np.array([[float(x) for x in r] for r in eM]), rtol=1e-12, atol=1e-12,
                  what=f"P-6 M {mode} nz={nz}")
            close(z[0, 0], np.array([float(x) for x in ez]), rtol=1e-14, atol=1e-14,
                  what=f"P-6 z {mode}")
    assert isinstance(Fraction(1, 3), Fraction)


def pin_p7_brute_force(ora):
    """Token-by-token scalar evaluation on tiny inputs with finite gates."""
    for shp, N, mode in [(dict(B=2, Hq=4, Hkv=2, L=7, dk=3, dv=2), N, mode)
                         for N in (3, 7) for mode in ("linear", "delta")] + [
            (dict(B=1, Hq=2, Hkv=1, L=5, dk=3, dv=3), 2, mode) for mode in ("linear", "delta")]:
        if True:
            c = case64(71 + N + shp["dv"], scale=1.4, nonzero_state=(N != 7), **shp)
            out, M, z = run(ora, c, N, mode)
            bo, bM, bz = ind.brute_force(c["q"], c["k"], c["v"], c["beta"], c["M0"], c["z0"], N,
                                         mode, c["eps"])
            close(out, bo, rtol=1e-11, atol=1e-12, what=f"P-7 out {mode} N={N}")
            close(M, bM, rtol=1e-11, atol=1e-12, what=f"P-7 M {mode} N={N}")
            close(z, bz, rtol=1e-13, atol=1e-13, what=f"P-7 z {mode} N={N}")


def pin_p8_gqa(ora):
    """Hq = g*Hkv equals MHA with K, V, M0, z0 repeated g times along heads;
    each copy of the state receives the same update."""
    for mode in ("linear", "delta"):
        c = case64(81, scale=1.3, nonzero_state=True, **SHAPE)
        out, M, z = run(ora, c, N_RAGGED, mode)
        g = SHAPE["Hq"] // SHAPE["Hkv"]
        rep = {k2: np.repeat(c[k2], g, axis=1) for k2 in ("k", "v", "M0", "z0")}
        c2 = dict(c, **rep)
        out2, M2, z2 = run(ora, c2, N_RAGGED, mode)
        close(out, out2, rtol=1e-13, atol=1e-14, what=f"P-8 out {mode}")
        close(np.repeat(M, g, axis=1), M2, rtol=1e-13, atol=1e-14, what=f"P-8 M {mode}")
        close(np.repeat(z, g, axis=1), z2, rtol=1e-13, atol=1e-14, what=f"P-8 z {mode}")


def pin_p9_split_calls(ora):
    """forward(L) == forward(L1) then forward(L - L1) with (M, z) carried over,
    for L1 a multiple of N: only (M, z) crosses segments."""
    shp = dict(SHAPE, L=14)
    for mode in ("linear", "delta"):
        c = case64(91, scale=1.3, **shp)
        out, M, z = run(ora, c, N_RAGGED, mode)
        L1 = 8
        c1 = dict(c, q=c["q"][:, :, :L1], k=c["k"][:, :, :L1], v=c["v"][:, :, :L1])
        o1, M1, z1 = run(ora, c1, N_RAGGED, mode)
        c2 = dict(c, q=c["q"][:, :, L1:], k=c["k"][:, :, L1:], v=c["v"][:, :, L1:], M0=M1, z0=z1)
        o2, M2, z2 = run(ora, c2, N_RAGGED, mode)
        close(np.concatenate([o1, o2], axis=2), out, rtol=1e-13, atol=1e-14, what=f"P-9 out {mode}")
        close(M2, M, rtol=1e-13, atol=1e-14, what=f"P-9 M {mode}")
        close(z2, z, rtol=1e-13, atol=1e-14, what=f"P-9 z {mode}")


def pin_p10_structure(ora):
    """Equivariance under a batch permutation and under a permutation of kv
    groups moved together with their query heads and gates; and with N = L and
    zero state, out = (1 - gamma) * full causal SDPA."""
    c = case64(101, scale=1.3, nonzero_state=True, **SHAPE)
    out, M, z = run(ora, c, N_RAGGED, "delta")
    pb = np.array([1, 0])
    cb = {k2: (c[k2][pb] if k2 in ("q", "k", "v", "M0", "z0") else c[k2]) for k2 in c}
    ob, Mb, zb = run(ora, cb, N_RAGGED, "delta")
    close(ob, out[pb], rtol=1e-14, atol=0, what="P-10 batch perm")
    close(Mb, M[pb], rtol=1e-14, atol=0, what="P-10 batch perm M")
    g = SHAPE["Hq"] // SHAPE["Hkv"]
    pk = np.array([2, 0, 1])
    pq = np.concatenate([np.arange(j * g, (j + 1) * g) for j in pk])
    ch = dict(c, q=c["q"][:, pq], beta=c["beta"][pq], k=c["k"][:, pk], v=c["v"][:, pk],
              M0=c["M0"][:, pk], z0=c["z0"][:, pk])
    oh, Mh, zh = run(ora, ch, N_RAGGED, "delta")
    close(oh, out[:, pq], rtol=1e-14, atol=0, what="P-10 head perm")
    close(Mh, M[:, pk], rtol=1e-14, atol=0, what="P-10 head perm M")
    c0 = case64(102, scale=1.3, **SHAPE)
    L = SHAPE["L"]
    o0, _, _ = run(ora, c0, L, "linear")
    gam = 1.0 / (1.0 + np.exp(-c0["beta"]))
    ref = (1.0 - gam)[None, :, None, None] * ind.sdpa_per_segment(c0["q"], c0["k"], c0["v"], L)
    close(o0, ref, rtol=1e-11, atol=1e-12, what="P-10 N=L")


def pin_p11_unit_segments(ora):
    """N = 1: each row attends only to itself, so A_dot = v exactly."""
    c = case64(111, scale=2.0, **SHAPE)
    out, _, _ = run(ora, c, 1, "linear", beta=np.full(SHAPE["Hq"], -INF))
    g = SHAPE["Hq"] // SHAPE["Hkv"]
    assert np.array_equal(out, np.repeat(c["v"], g, axis=1)), "P-11: A_dot != v at N=1"


def pin_p12_delta_affine(ora):
    """Delta rule as an affine map: M_s = (I - G_s) M_{s-1} + H_s with
    G_s = sig(K)^T diag(1/(sig(K) z + eps)) sig(K) and H_s = sig(K)^T V."""
    rng = np.random.default_rng(121)
    dk, dv, n = 5, 3, 9
    for _ in range(3):
        M = rng.standard_normal((dk, dv))
        z = np.abs(rng.standard_normal(dk)) * 5.0 + 0.1
        ks = rng.standard_normal((n, dk)) * 1.5
        vs = rng.standard_normal((n, dv))
        sk = np.where(ks > 0, ks + 1.0, np.exp(np.minimum(ks, 0.0)))
        G = sk.T @ (sk / (sk @ z + 1e-6)[:, None])
        H = sk.T @ vs
        M2, _ = ora.memory_update(ks, vs, M, z, "delta", 1e-6)
        close(M2, (np.eye(dk) - G) @ M + H, rtol=1e-11, atol=1e-12, what="P-12")


def pin_p13_streaming(ora):
    """Streaming decode (chunks of 1, 2 or 3 rows, and whole segments) equals
    the token-by-token brute force: outputs, and the state after the stream
    (the last, unfinished segment written at the end)."""
    for shp, N, mode, chunk in [(dict(B=2, Hq=4, Hkv=2, L=7, dk=3, dv=2), 3, m, c)
                                for m in ("linear", "delta") for c in (1, 2, 3)] + [
            (dict(B=1, Hq=2, Hkv=1, L=5, dk=3, dv=3), 2, "delta", 2)]:
        c = case64(131 + N + chunk, scale=1.4, nonzero_state=True, **shp)
        out, M, z = ora.streaming_decode(c["q"], c["k"], c["v"], c["beta"], c["M0"], c["z0"], N,
                                         mode, chunk, c["eps"])
        bo, bM, bz = ind.brute_force(c["q"], c["k"], c["v"], c["beta"], c["M0"], c["z0"], N,
                                     mode, c["eps"])
        tag = f"P-13 {mode} N={N} chunk={chunk}"
        close(out, bo, rtol=1e-11, atol=1e-12, what=f"{tag} out")
        close(M, bM, rtol=1e-11, atol=1e-12, what=f"{tag} M")
        close(z, bz, rtol=1e-13, atol=1e-13, what=f"{tag} z")


def pin_p14_block(ora):
    """The block equals scalar projections (explicit sums over d_model, head h
    = columns h*d .. h*d + d - 1) around the token-by-token brute force, then
    the scalar output projection over (head, column) pairs. d_model differs
    from Hq * d, so a transposed weight or a wrong head split cannot pass."""
    rng = np.random.default_rng(141)
    for B, L, dm, Hq, Hkv, d, N, mode in [(2, 5, 4, 2, 1, 3, 3, "delta"),
                                          (1, 6, 5, 2, 2, 2, 4, "linear")]:
        x = rng.standard_normal((B, L, dm))
        wq = rng.standard_normal((dm, Hq * d)) / math.sqrt(dm)
        wk = rng.standard_normal((dm, Hkv * d)) / math.sqrt(dm)
        wv = rng.standard_normal((dm, Hkv * d)) / math.sqrt(dm)
        wo = rng.standard_normal((Hq * d, dm)) / math.sqrt(Hq * d)
        beta = rng.standard_normal(Hq)
        M0 = 0.1 * rng.standard_normal((B, Hkv, d, d))
        z0 = rng.uniform(0.5, 2.0, (B, Hkv, d))
        y, M, z = ora.infini_block(x, wq, wk, wv, wo, beta, M0, z0, N, mode, Hq, Hkv, 1e-6)

        def proj(w, n):
            out = np.zeros((B, n, L, d))
            for b in range(B):
                for h in range(n):
                    for l in range(L):
                        for c in range(d):
                            acc = 0.0
                            for i in range(dm):
                                acc += x[b, l, i] * w[i, h * d + c]
                            out[b, h, l, c] = acc
            return out

        q, k, v = proj(wq, Hq), proj(wk, Hkv), proj(wv, Hkv)
        bo, bM, bz = ind.brute_force(q, k, v, beta, M0, z0, N, mode, 1e-6)
        by = np.zeros((B, L, dm))
        for b in range(B):
            for l in range(L):
                for j in range(dm):
                    acc = 0.0
                    for h in range(Hq):
                        for c in range(d):
                            acc += bo[b, h, l, c] * wo[h * d + c, j]
                    by[b, l, j] = acc
        tag = f"P-14 {mode} dm={dm} Hq={Hq} d={d}"
        close(y, by, rtol=1e-10, atol=1e-12, what=f"{tag} y")
        close(M, bM, rtol=1e-10, atol=1e-12, what=f"{tag} M")
        close(z, bz, rtol=1e-12, atol=1e-12, what=f"{tag} z")


def _loss(ora, c, N, mode, d_out, d_M, d_z):
    out, M, z = ora.infini_attention(c["q"], c["k"], c["v"], c["beta"], c["M0"], c["z0"], N,
                                     mode, c["eps"])
    return float(np.sum(d_out * out) + np.sum(d_M * M) + np.sum(d_z * z))


def pin_p15_backward_finite_differences(ora):
    """The backward pass through time equals central finite differences of the
    forward's scalar loss <d_out, out> + <d_M, M_S> + <d_z, z_S>, for every
    element of q, k, v, beta, M0 and z0 (several segments, grouped heads,
    both rules); at beta = +-inf the gate's gradient is exactly 0."""
    h = 1e-5
    for shp, N, mode in [(dict(B=1, Hq=2, Hkv=1, L=5, dk=3, dv=3), 2, "delta"),
                         (dict(B=1, Hq=2, Hkv=1, L=5, dk=3, dv=3), 2, "linear"),
                         (dict(B=2, Hq=2, Hkv=2, L=4, dk=2, dv=2), 3, "delta")]:
        c = case64(151 + N + shp["B"], scale=1.2, nonzero_state=True, **shp)
        rng = np.random.default_rng(152 + N)
        d_out = rng.standard_normal((shp["B"], shp["Hq"], shp["L"], shp["dv"]))
        d_M = rng.standard_normal(c["M0"].shape)
        d_z = rng.standard_normal(c["z0"].shape)
        grads = ora.infini_attention_backward(c["q"], c["k"], c["v"], c["beta"], c["M0"],
                                              c["z0"], N, mode, d_out, d_M, d_z, c["eps"])
        for name, g in zip(("q", "k", "v", "beta", "M0", "z0"), grads):
            fd = np.zeros_like(c[name])
            for idx in np.ndindex(*c[name].shape):
                orig = c[name][idx]
                c[name][idx] = orig + h
                up = _loss(ora, c, N, mode, d_out, d_M, d_z)
                c[name][idx] = orig - h
                dn = _loss(ora, c, N, mode, d_out, d_M, d_z)
                c[name][idx] = orig
                fd[idx] = (up - dn) / (2 * h)
            close(g, fd, rtol=1e-6, atol=1e-7, what=f"P-15 d{name} {mode} N={N}")
        # gates at the infinities: no gradient into beta
        inf_beta = np.array([INF, -INF])
        g = ora.infini_attention_backward(c["q"], c["k"], c["v"], inf_beta, c["M0"], c["z0"], N,
                                          mode, d_out, d_M, d_z, c["eps"])
        assert np.all(g[3] == 0.0), "P-15: gradient into an infinite gate"


def pin_p16_memory_chain(ora):
    """The (M, z) recurrence on its own (``memory_chain``, which the full-size
    state comparisons use as their only reference) equals the token-by-token
    brute force's final state, and each state it keeps equals the brute
    force's final state over the rows before that segment; under the linear
    rule it also equals the closed form sum sig(k)^T v, sum sig(k). Checked on
    fp64 inputs and on bf16-stored inputs streamed through ``upcast``, with a
    ragged last segment, under both rules."""
    from synth import round_bf16_bits, round_fp32
    shp = dict(B=2, Hq=4, Hkv=2, L=11, dk=3, dv=4)
    N = 4  # segments of 4, 4, 3
    for mode in ("linear", "delta"):
        c = case64(161, scale=1.3, nonzero_state=True, **shp)
        kb = round_bf16_bits(round_fp32(c["k"]))
        vb = round_bf16_bits(round_fp32(c["v"]))
        variants = [("fp64", c["k"], c["v"], None),
                    ("bf16", kb, vb, lambda a: as_f64(a, "bf16"))]
        for tag, k, v, up in variants:
            kf = c["k"] if up is None else as_f64(kb, "bf16")
            vf = c["v"] if up is None else as_f64(vb, "bf16")
            _, bM, bz = ind.brute_force(c["q"], kf, vf, c["beta"], c["M0"], c["z0"], N, mode,
                                        c["eps"])
            for b in range(shp["B"]):
                for j in range(shp["Hkv"]):
                    M, z, states = ora.memory_chain(k[b, j], v[b, j], c["M0"][b, j],
                                                    c["z0"][b, j], N, mode, c["eps"],
                                                    keep_states=True, upcast=up)
                    what = f"P-16 {mode} {tag} b{b} j{j}"
                    close(M, bM[b, j], rtol=1e-11, atol=1e-12, what=f"{what} M_S")
                    close(z, bz[b, j], rtol=1e-13, atol=1e-13, what=f"{what} z_S")
                    if mode == "linear":
                        sk = np.where(kf[b, j] > 0, kf[b, j] + 1.0,
                                      np.exp(np.minimum(kf[b, j], 0.0)))
                        close(M, c["M0"][b, j] + sk.T @ vf[b, j], rtol=1e-12, atol=1e-12,
                              what=f"{what} closed-form M")
                        close(z, c["z0"][b, j] + sk.sum(axis=0), rtol=1e-13, atol=1e-13,
                              what=f"{what} closed-form z")
                    starts = list(range(0, shp["L"], N))
                    assert len(states) == len(starts), f"{what}: {len(states)} states"
                    for s, a in enumerate(starts):
                        if a == 0:
                            pM, pz = c["M0"][b, j], c["z0"][b, j]
                        else:
                            sub = dict(q=c["q"][:, :, :a], k=kf[:, :, :a], v=vf[:, :, :a])
                            _, pMs, pzs = ind.brute_force(sub["q"], sub["k"], sub["v"],
                                                          c["beta"], c["M0"], c["z0"], N, mode,
                                                          c["eps"])
                            pM, pz = pMs[b, j], pzs[b, j]
                        close(states[s][0], pM, rtol=1e-11, atol=1e-12, what=f"{what} M_{s-1}")
                        close(states[s][1], pz, rtol=1e-13, atol=1e-13, what=f"{what} z_{s-1}")


ALL_PINS = [
    pin_sigma_library, pin_gate_library, pin_golden, pin_p1_sdpa, pin_p2_dense_linear,
    pin_p3_linear_closed_form, pin_p4_zero_start, pin_p5_delta_fixed_point, pin_p6_exact,
    pin_p7_brute_force, pin_p8_gqa, pin_p9_split_calls, pin_p10_structure,
    pin_p11_unit_segments, pin_p12_delta_affine, pin_p13_streaming,
    pin_p14_block, pin_p15_backward_finite_differences, pin_p16_memory_chain,
]
