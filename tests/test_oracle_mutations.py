"""Planted mistakes in the oracle (on the CPU) must each be caught by a pin.

Every mutant below is a plausible slip when writing the oracle from the
slides: a dropped latent term, a wrong head index, a swapped K/V factor, a
sign error, a wrong scale, a missing normalisation, an off-by-one length or
causal mask.  The mutation is applied to the oracle module in-process; the
real oracle is restored after each case.
"""
import math

import numpy as np
import pytest

import oracle.lrkv_oracle as O
from tests import oracle_pins as P
from tests.test_oracle_pins import tiny_inputs

_orig_implied = O.implied_kv
_orig_softmax = O.softmax_attention
_orig_decode = O.decode
_orig_prefill = O.prefill
_orig_projected = O.projected_rows


def _implied(fk=None, fv=None):
    def mutant(k_s, v_s, z_k, z_v, b_k, b_v):
        k_s, v_s, z_k, z_v, b_k, b_v = (np.asarray(a, np.float64) for a in (k_s, v_s, z_k, z_v, b_k, b_v))
        H = b_k.shape[0]
        K = np.stack([fk(k_s, z_k, b_k, b_v, h) if fk else k_s + z_k[:, h] @ b_k[h].T for h in range(H)])
        V = np.stack([fv(v_s, z_v, b_k, b_v, h) if fv else v_s + z_v[:, h] @ b_v[h].T for h in range(H)])
        return K, V
    return mutant


def _softmax(kind):
    def mutant(q, K, V, scale):
        if K.shape[0] == 0:
            return np.zeros(V.shape[1])
        if kind == "scale_squared":
            scale = scale * scale
        s = (K @ q) * scale
        e = np.exp(s - s.max())
        if kind == "unnormalised":
            return e @ V
        return (e / e.sum()) @ V
    return mutant


def _decode_len(delta):
    def mutant(q, k_s, v_s, z_k, z_v, b_k, b_v, seq_lens, scale=None):
        lens = [max(0, min(int(L) + delta, k_s.shape[1])) for L in seq_lens]
        return _orig_decode(q, k_s, v_s, z_k, z_v, b_k, b_v, lens, scale)
    return mutant


def _prefill_mask(k):
    def mutant(q, k_s, v_s, z_k, z_v, b_k, b_v, scale=None):
        q = np.asarray(q, np.float64)
        B, L, H, d_h = q.shape
        sc = 1.0 / math.sqrt(d_h)
        out = np.zeros((B, L, H, d_h))
        masked = np.triu(np.ones((L, L), bool), k=k) if k is not None else np.zeros((L, L), bool)
        for b in range(B):
            K, V = O.implied_kv(k_s[b], v_s[b], z_k[b], z_v[b], b_k, b_v)
            for h in range(H):
                S = (q[b, :, h] @ K[h].T) * sc
                S[masked] = -1e300
                E = np.exp(S - S.max(axis=1, keepdims=True))
                out[b, :, h] = (E / E.sum(axis=1, keepdims=True)) @ V[h]
        return out
    return mutant


def _past(kind):
    def mutant(q, k_s, v_s, z_k, z_v, b_k, b_v, start, scale=None):
        q = np.asarray(q, np.float64)
        B, L, H, d_h = q.shape
        out = np.zeros((B, L, H, d_h))
        for b in range(B):
            s0 = 0 if kind == "ignored" else int(start[b])
            n = s0 + L
            K, V = O.implied_kv(k_s[b, :n], v_s[b, :n], z_k[b, :n], z_v[b, :n], b_k, b_v)
            pos = s0 + np.arange(L)[:, None]
            masked = np.arange(n)[None, :] >= pos if kind == "excludes_diagonal" else np.arange(n)[None, :] > pos
            for h in range(H):
                S = (q[b, :, h] @ K[h].T) / math.sqrt(d_h)
                S[masked] = -1e300
                E = np.exp(S - S.max(axis=1, keepdims=True))
                out[b, :, h] = (E / E.sum(axis=1, keepdims=True)) @ V[h]
        return out
    return mutant


def _count_without_heads(mechanism, *, d_h, H=1, r=0, n_kv=1, layers=1):
    if mechanism == "lrkv":
        return 2 * (d_h + r) * layers
    return _orig_count(mechanism, d_h=d_h, H=H, r=r, n_kv=n_kv, layers=layers)


_orig_count = O.cache_elems_per_token


def _projected(kind):
    def mutant(X, Wk_shared, Wv_shared, Uk, Uv):
        if kind == "kv_swapped":
            return _orig_projected(X, Wv_shared, Wk_shared, Uk, Uv)
        Uk_shift = np.roll(np.asarray(Uk), 1, axis=0)           # head h takes U of head h - 1
        return _orig_projected(X, Wk_shared, Wv_shared, Uk_shift, Uv)
    return mutant

_orig_backward = O.prefill_backward
_orig_lse = O.prefill_forward_lse


def _backward(kind):
    """The oracle's backward pass with one planted slip."""
    def mutant(q, k_s, v_s, z_k, z_v, b_k, b_v, d_out, scale=None):
        q, d_out, z_k, z_v, b_k, b_v = (np.asarray(a, np.float64) for a in (q, d_out, z_k, z_v, b_k, b_v))
        B, L, H, d_h = q.shape
        r = b_k.shape[2]
        sc = 1.0 / math.sqrt(d_h)
        g = {"dq": np.zeros_like(q), "dk_s": np.zeros((B, L, d_h)), "dv_s": np.zeros((B, L, d_h)),
             "dz_k": np.zeros((B, L, H, r)), "dz_v": np.zeros((B, L, H, r)),
             "db_k": np.zeros((H, d_h, r)), "db_v": np.zeros((H, d_h, r))}
        future = np.triu(np.ones((L, L), dtype=bool), k=1)
        for b in range(B):
            K, V = O.implied_kv(k_s[b], v_s[b], z_k[b], z_v[b], b_k, b_v)
            for h in range(H):
                Qh, dO = q[b, :, h, :], d_out[b, :, h, :]
                S = (Qh @ K[h].T) * sc
                S[future] = -np.inf
                E = np.exp(S - S.max(axis=1, keepdims=True))
                A = E / E.sum(axis=1, keepdims=True)
                dV = A.T @ dO
                dA = dO @ V[h].T
                dS = A * dA if kind == "no_softmax_rowsum" else A * (dA - (A * dA).sum(axis=1, keepdims=True))
                g["dq"][b, :, h, :] = sc * (dS @ (V[h] if kind == "dq_uses_values" else K[h]))
                dK = (1.0 if kind == "dk_without_scale" else sc) * (dS.T @ Qh)
                g["dk_s"][b] += dK
                g["dv_s"][b] += dV
                g["dz_k"][b, :, h, :] = dK @ (b_v[h] if kind == "dz_k_uses_value_factor" else b_k[h])
                g["dz_v"][b, :, h, :] = dV @ b_v[h]
                g["db_k"][h] += dK.T @ z_k[b, :, h, :]
                g["db_v"][h] += dV.T @ z_v[b, :, h, :]
        return g
    return mutant


def _lse_mutant(q, k_s, v_s, z_k, z_v, b_k, b_v, scale=None):
    out, lse = _orig_lse(q, k_s, v_s, z_k, z_v, b_k, b_v, scale)
    return out, lse / math.log(2.0)          # log2 where the natural log is meant


MUTANTS = {
    "lrkv_count_without_heads": ("cache_elems_per_token", _count_without_heads),
    "drop_key_latent": ("implied_kv", _implied(fk=lambda k, z, bk, bv, h: k)),
    "drop_value_latent": ("implied_kv", _implied(fv=lambda v, z, bk, bv, h: v)),
    "key_factor_of_head0": ("implied_kv", _implied(fk=lambda k, z, bk, bv, h: k + z[:, h] @ bk[0].T)),
    "key_uses_value_factor": ("implied_kv", _implied(fk=lambda k, z, bk, bv, h: k + z[:, h] @ bv[h].T)),
    "latent_sign_flipped": ("implied_kv", _implied(fv=lambda v, z, bk, bv, h: v - z[:, h] @ bv[h].T)),
    "latent_of_next_head": ("implied_kv", _implied(
        fk=lambda k, z, bk, bv, h: k + z[:, (h + 1) % z.shape[1]] @ bk[h].T)),
    "scale_one_over_d": ("softmax_attention", _softmax("scale_squared")),
    "unnormalised_softmax": ("softmax_attention", _softmax("unnormalised")),
    "length_minus_one": ("decode", _decode_len(-1)),
    "length_plus_one": ("decode", _decode_len(+1)),
    "causal_mask_excludes_diagonal": ("prefill", _prefill_mask(0)),
    "no_causal_mask": ("prefill", _prefill_mask(None)),
    "causal_mask_one_ahead": ("prefill", _prefill_mask(2)),
    "past_ignored": ("prefill_with_past", _past("ignored")),
    "past_mask_excludes_diagonal": ("prefill_with_past", _past("excludes_diagonal")),
    "projection_kv_swapped": ("projected_rows", _projected("kv_swapped")),
    "projection_latent_of_previous_head": ("projected_rows", _projected("head_shift")),
    "backward_no_softmax_rowsum": ("prefill_backward", _backward("no_softmax_rowsum")),
    "backward_dq_uses_values": ("prefill_backward", _backward("dq_uses_values")),
    "backward_dk_without_scale": ("prefill_backward", _backward("dk_without_scale")),
    "backward_dz_k_uses_value_factor": ("prefill_backward", _backward("dz_k_uses_value_factor")),
    "lse_in_log2": ("prefill_forward_lse", _lse_mutant),
}


def _run_all_pins():
    caught = []
    checks = list(P.ALL_PINS) + [lambda O_: P.pin_decode_brute_force(O_, tiny_inputs()),
                                 lambda O_: P.pin_weight_level_on_tiny_workload(O_, tiny_inputs())]
    for pin in checks:
        try:
            pin(O)
        except (AssertionError, ValueError, IndexError) as e:  # noqa: PERF203
            caught.append(getattr(pin, "__name__", "lambda"))
    return caught


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(O, attr, fn)
    caught = _run_all_pins()
    assert caught, f"planted mistake {name!r} passed every pin"


def test_unmutated_oracle_passes_every_pin():
    assert _run_all_pins() == []
