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
                                       "memory_update", "infini_attention")}


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
