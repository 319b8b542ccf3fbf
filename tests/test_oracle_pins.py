"""The fp64 oracle against its pins, and planted mistakes against the pins."""

import math

import numpy as np
import pytest

import oracle.infini_ref as ref
import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(ref)


# ---------------------------------------------------------------------------
# Planted mistakes (in the oracle, on the CPU): each must be caught by a pin.
# ---------------------------------------------------------------------------

_orig = {n: getattr(ref, n) for n in ("elu_plus_one", "gate_value", "kv_head_of",
                                       "local_causal_attention", "memory_retrieval",
                                       "memory_update", "infini_attention",
                                       "streaming_decode", "infini_block",
                                       "infini_attention_backward", "_elu_plus_one_grad",
                                       "memory_chain")}


def _retrieval_no_eps(qs, M, z, eps):
    sq = ref.elu_plus_one(qs)
    return (sq @ M) / (sq @ z)[:, None]


def _retrieval_scaled_q(qs, M, z, eps):
    sq = ref.elu_plus_one(qs / math.sqrt(qs.shape[1]))
    return (sq @ M) / (sq @ z + eps)[:, None]


def _retrieval_transposed(qs, M, z, eps):
    sq = ref.elu_plus_one(qs)
    return (sq @ M.T) / (sq @ z + eps)[:, None]


def _update_factory(variant):
    def upd(ks, vs, M, z, mode, eps):
        sk = ref.elu_plus_one(ks)
        if mode == "linear":
            write = vs
        else:
            den = sk @ z + (0.0 if variant == "delta_no_eps" else eps)
            r = (sk @ M) / den[:, None]
            write = vs + r if variant == "delta_sign" else vs - r
        if variant == "keys_as_values":
            return M + sk.T @ ks, z + sk.sum(0)
        if variant == "no_z":
            return M + sk.T @ write, z
        if variant == "delta_new_z" and mode == "delta":
            z2 = z + sk.sum(0)
            r = (sk @ M) / (sk @ z2 + eps)[:, None]
            return M + sk.T @ (vs - r), z2
        return M + sk.T @ write, z + sk.sum(0)
    return upd


def _attn_no_scale(qs, ks, vs):
    n = qs.shape[0]
    s = qs @ ks.T
    s = np.where(np.triu(np.ones((n, n), bool), 1), -np.inf, s)
    p = np.exp(s - s.max(1, keepdims=True))
    return (p / p.sum(1, keepdims=True)) @ vs


def _attn_mask_shift(qs, ks, vs):
    n, dk = qs.shape
    s = qs @ ks.T / math.sqrt(dk)
    s = np.where(np.triu(np.ones((n, n), bool), 2), -np.inf, s)
    p = np.exp(s - s.max(1, keepdims=True))
    return (p / p.sum(1, keepdims=True)) @ vs


def _update_before_retrieval(q, k, v, beta, M0, z0, seg_len, mode, eps=1e-6):
    B, Hq, L, dk = q.shape
    Hkv, dv = k.shape[1], v.shape[3]
    gam = ref.gate_value(beta)
    M, z = M0.copy(), z0.copy()
    out = np.empty((B, Hq, L, dv))
    for a, e in ref.segment_bounds(L, seg_len):
        for b in range(B):
            for j in range(Hkv):
                M[b, j], z[b, j] = ref.memory_update(k[b, j, a:e], v[b, j, a:e], M[b, j], z[b, j],
                                                     mode, eps)
        for b in range(B):
            for h in range(Hq):
                j = ref.kv_head_of(h, Hq, Hkv)
                ad = ref.local_causal_attention(q[b, h, a:e], k[b, j, a:e], v[b, j, a:e])
                am = ref.memory_retrieval(q[b, h, a:e], M[b, j], z[b, j], eps)
                out[b, h, a:e] = gam[h] * am + (1 - gam[h]) * ad
    return out, M, z


def _stream_factory(variant):
    """streaming_decode with one step of the stream done wrong."""
    def stream(q, k, v, beta, M0, z0, seg_len, mode, chunk=1, eps=1e-6):
        B, Hq, L, dk = q.shape
        Hkv = k.shape[1]
        gamma = ref.gate_value(beta)
        M, z = np.array(M0, dtype=np.float64), np.array(z0, dtype=np.float64)
        out = np.empty((B, Hq, L, v.shape[3]))
        ck, cv, n, t = [], [], 0, 0
        while t < L:
            m = min(chunk, seg_len - n, L - t)
            for r in range(m):
                for b in range(B):
                    for h in range(Hq):
                        j = ref.kv_head_of(h, Hq, Hkv)
                        keys = np.array([x[b, j] for x in ck] + [k[b, j, t + r]])
                        vals = np.array([x[b, j] for x in cv] + [v[b, j, t + r]])
                        if variant == "exclusive" and len(keys) > 1:
                            keys, vals = keys[:-1], vals[:-1]
                        row = q[b, h, t + r][None]
                        a_dot = ref.local_causal_attention_rows(row, np.array([len(keys) - 1]),
                                                                keys, vals)
                        a_mem = ref.memory_retrieval(row, M[b, j], z[b, j], eps)
                        out[b, h, t + r] = gamma[h] * a_mem[0] + (1 - gamma[h]) * a_dot[0]
                ck.append(k[:, :, t + r]); cv.append(v[:, :, t + r])
            n += m
            t += m
            if n == seg_len or t == L or variant == "update_every_chunk":
                start = len(ck) - (m if variant == "update_every_chunk" else n)
                for b in range(B):
                    for j in range(Hkv):
                        ks = np.array([x[b, j] for x in ck[start:]])
                        vs = np.array([x[b, j] for x in cv[start:]])
                        M[b, j], z[b, j] = ref.memory_update(ks, vs, M[b, j], z[b, j], mode, eps)
                if n == seg_len or t == L:
                    ck, cv, n = [], [], 0
        return out, M, z
    return stream


def _block_factory(variant):
    """infini_block with its layout done wrong."""
    def block(x, wq, wk, wv, wo, beta, M0, z0, seg_len, mode, n_q_heads, n_kv_heads, eps=1e-6):
        B, L, dm = x.shape
        d = wq.shape[1] // n_q_heads

        def heads(w, n):
            if variant == "column_major_heads":  # head h = columns h, h + n, h + 2n, ...
                return (x @ w).reshape(B, L, d, n).transpose(0, 3, 1, 2)
            return (x @ w).reshape(B, L, n, d).transpose(0, 2, 1, 3)

        q, k, v = heads(wq, n_q_heads), heads(wk, n_kv_heads), heads(wv, n_kv_heads)
        out, M, z = ref.infini_attention(q, k, v, beta, M0, z0, seg_len, mode, eps)
        if variant == "heads_regrouped_wrong":
            y = out.transpose(0, 2, 3, 1).reshape(B, L, n_q_heads * d) @ wo
        else:
            y = out.transpose(0, 2, 1, 3).reshape(B, L, n_q_heads * d) @ wo
        return y, M, z
    return block


def _backward_with(old, new):
    """The oracle's backward with one line of its source replaced."""
    import inspect
    import textwrap
    src = textwrap.dedent(inspect.getsource(_orig["infini_attention_backward"]))
    assert src.count(old) == 1, old
    ns = dict(vars(ref))
    exec(compile(src.replace(old, new), "<planted>", "exec"), ns)
    return ns["infini_attention_backward"]


def _chain_with(old, new):
    """The oracle's memory_chain with one line of its source replaced."""
    import inspect
    import textwrap
    src = textwrap.dedent(inspect.getsource(_orig["memory_chain"]))
    assert src.count(old) == 1, old
    ns = dict(vars(ref))
    exec(compile(src.replace(old, new), "<planted>", "exec"), ns)
    return ns["memory_chain"]


def _chain_pre_last_state(k, v, M0, z0, seg_len, mode, eps=1e-6, keep_states=False, upcast=None):
    """Returns the state before the last segment instead of after it."""
    M, z, states = _orig["memory_chain"](k, v, M0, z0, seg_len, mode, eps, True, upcast)
    return states[-1][0], states[-1][1], (states if keep_states else None)


MUTANTS = {
    "no_eps_retrieval": ("memory_retrieval", _retrieval_no_eps),
    "sigma_on_scaled_q": ("memory_retrieval", _retrieval_scaled_q),
    "delta_sign": ("memory_update", _update_factory("delta_sign")),
    "delta_no_eps": ("memory_update", _update_factory("delta_no_eps")),
    "delta_new_z": ("memory_update", _update_factory("delta_new_z")),
    "update_writes_keys": ("memory_update", _update_factory("keys_as_values")),
    "retrieval_transposed_M": ("memory_retrieval", _retrieval_transposed),
    "no_z_update": ("memory_update", _update_factory("no_z")),
    "gate_swapped": ("gate_value", lambda b: 1.0 - _orig["gate_value"](b)),
    "no_softmax_scale": ("local_causal_attention", _attn_no_scale),
    "mask_off_by_one": ("local_causal_attention", _attn_mask_shift),
    "elu_without_plus_one": ("elu_plus_one", lambda x: _orig["elu_plus_one"](x) - 1.0),
    "gqa_modulo": ("kv_head_of", lambda h, hq, hkv: h % hkv),
    "update_before_retrieval": ("infini_attention", _update_before_retrieval),
    "stream_row_misses_itself": ("streaming_decode", _stream_factory("exclusive")),
    "stream_updates_every_chunk": ("streaming_decode", _stream_factory("update_every_chunk")),
    "block_heads_interleaved": ("infini_block", _block_factory("column_major_heads")),
    "block_output_regrouped_wrong": ("infini_block", _block_factory("heads_regrouped_wrong")),
    "backward_sigma_grad_one": ("_elu_plus_one_grad", lambda x: np.ones_like(x)),
    "backward_sigma_grad_exp": ("_elu_plus_one_grad", lambda x: np.exp(x)),
    "backward_delta_sign": ("infini_attention_backward", _backward_with("dR = -dW", "dR = dW")),
    "backward_retrieval_no_den_term": ("infini_attention_backward", _backward_with(
        "dden = -np.sum(dAm * num, axis=1) / den ** 2", "dden = 0.0 * den")),
    "backward_drops_z_carry": ("infini_attention_backward", _backward_with(
        "gMp, gzp = gM.copy(), gz.copy()", "gMp, gzp = gM.copy(), np.zeros_like(gz)")),
    "chain_returns_pre_last_state": ("memory_chain", _chain_pre_last_state),
    "chain_keeps_states_after_update": ("memory_chain", _chain_with(
        "M, z = memory_update(ks, vs, M, z, mode, eps)",
        "M, z = memory_update(ks, vs, M, z, mode, eps)\n        if keep_states:\n"
        "            states[-1] = (M.copy(), z.copy())")),
    "chain_skips_last_segment": ("memory_chain", _chain_with(
        "for (a, e) in segment_bounds(L, seg_len):", "for (a, e) in segment_bounds(L, seg_len)[:-1]:")),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(ref, attr, fn)
    caught = []
    with np.errstate(all="ignore"):
        for pin in pins.ALL_PINS:
            try:
                pin(ref)
            except Exception as exc:  # noqa: BLE001 - any failure counts as caught
                caught.append((pin.__name__, type(exc).__name__))
    assert caught, f"planted mistake {name!r} passed every pin"
