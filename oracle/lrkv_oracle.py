"""Float64 CPU oracle for attention over an LRKV compressed KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, links or runs
this module: only the tests, the smoke check of ``__graft_entry__`` and the
CPU-baseline leg of ``bench.py`` may use it.  It shares no code with the HIP
library and never touches a GPU.

Source: *Low-Rank Key Value Attention* (O'Neill, Clancy, Matskevichus, Reid,
arXiv:2601.11471v3), as restated in the independent slide discussion of that
paper.  Slides are cited by their frame title, with the paper equation or
table they restate.

What is computed is the plain definition, not the fast form: every head's
keys and values are reconstructed explicitly from the cache (or from the
weights), then ordinary softmax attention runs on them.  The absorbed form
that the kernels use (slides "Compute logits without expanding historical
keys", Eq. (6), and "Aggregate values before the residual up-projection",
Eq. (7)) is exact for the linear model, so it must reach the same result up
to rounding; the pins in ``tests/`` check that independently.

Notation (column form; the slides use row vectors, the two are transposes):
  H heads of width d_h, residual rank r, d = H * d_h.
  Cache per sequence: K_s, V_s  [T, d_h]; latents R^K, R^V  [T, H, r].
  Weights per head:   B^K_h, B^V_h  [d_h, r]   (stored as [H, d_h, r]).
  Implied key of head h at token t:  k_{h,t} = k_{s,t} + B^K_h z^K_{t,h}.

Readings of points the pages leave open (each is stated where it is used):
  * scale: 1/sqrt(d_h) on the sum of both score paths (the dotted vectors
    q_h and K_h are d_h wide);
  * decode masking: the query attends to every cached token of its sequence
    (the current token is appended before decoding), so nothing inside the
    cache is masked; prefill query i sees keys j <= i; with start cached
    tokens in front (a prefill chunk), new token i sees keys j <= start + i;
  * an empty sequence (length 0) yields an all-zero output;
  * no position encoding and no normalisation inside attention.

Every function here is pinned by the not-gpu tests (printed numbers, closed
forms, library routines, brute force); none is "parity unpinned".
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

__all__ = [
    "cache_elems_per_token", "cache_ratio_vs_mha", "kv_param_count",
    "head_projections", "cache_from_inputs", "implied_kv", "softmax_attention",
    "decode", "prefill", "prefill_with_past", "decode_from_weights", "append", "projected_rows",
    "prefill_forward_lse", "prefill_backward",
]


# ---------------------------------------------------------------------------
# Cache accounting.
# Slide "Can heads share storage while keeping distinct K/V features?"
# (paper Secs. 1-3): elements per token per layer are MHA 2*H*d_h,
# MQA 2*d_h, GQA 2*n_kv*d_h, LRKV 2*(d_h + H*r).  Multiplying by the layer
# count gives the per-token total over a model.
# ---------------------------------------------------------------------------
def cache_elems_per_token(mechanism: str, *, d_h: int, H: int = 1, r: int = 0,
                          n_kv: int = 1, layers: int = 1) -> int:
    mechanism = mechanism.lower()
    if mechanism == "mha":
        per_layer = 2 * H * d_h
    elif mechanism == "mqa":
        per_layer = 2 * d_h
    elif mechanism == "gqa":
        per_layer = 2 * n_kv * d_h
    elif mechanism == "lrkv":
        per_layer = 2 * (d_h + H * r)
    else:
        raise ValueError(f"unknown mechanism {mechanism!r}")
    return per_layer * layers


def cache_ratio_vs_mha(H: int, d_h: int, r: int) -> float:
    """LRKV cache over MHA cache for the same (H, d_h): the first form of
    slide "The rank directly sets the theoretical cache budget", Eq. (9),
    i.e. the ratio of the two element counts (L cancels)."""
    return cache_elems_per_token("lrkv", d_h=d_h, H=H, r=r) / cache_elems_per_token("mha", d_h=d_h, H=H)


def kv_param_count(mechanism: str, *, d: int, d_h: int, H: int, r: int = 0) -> int:
    """K/V projection parameter counts, slide "Smaller storage trades bandwidth
    for extra arithmetic", Eq. (10): LRKV has two shared d x d_h matrices plus
    per head U_h (d x r) and B_h (d_h x r) for K and for V; MHA has 2*H*d*d_h."""
    if mechanism == "lrkv":
        shared = 2 * d * d_h
        residual = 2 * H * (d * r + d_h * r)
        return shared + residual
    if mechanism == "mha":
        return 2 * H * d * d_h
    raise ValueError(mechanism)


# ---------------------------------------------------------------------------
# Weight-level model.
# Slide "LRKV constrains differences between heads", Eqs. (2)-(3):
#   W_h = W_shared + U_h B_h^T,  W_shared in R^{d x d_h}, U_h in R^{d x r},
#   B_h in R^{d_h x r}, separate factors for K and for V.
# ---------------------------------------------------------------------------
def head_projections(W_shared: np.ndarray, U: np.ndarray, Bf: np.ndarray) -> np.ndarray:
    """Explicit per-head projections W_h = W_shared + U_h B_h^T  ->  [H, d, d_h]."""
    W_shared = np.asarray(W_shared, np.float64)
    U = np.asarray(U, np.float64)
    Bf = np.asarray(Bf, np.float64)
    H = U.shape[0]
    return np.stack([W_shared + U[h] @ Bf[h].T for h in range(H)])


def cache_from_inputs(X: np.ndarray, W_shared: np.ndarray, U: np.ndarray):
    """What the cache stores for inputs X [L, d]: the shared features
    X W_shared [L, d_h] and the per-head latents X U_h, returned as [L, H, r].
    Slide "Cache shared features and compact per-head latents", Eqs. (4)-(5)."""
    X = np.asarray(X, np.float64)
    shared = X @ np.asarray(W_shared, np.float64)
    latents = np.stack([X @ np.asarray(U[h], np.float64) for h in range(U.shape[0])], axis=1)
    return shared, latents


def projected_rows(X, Wk_shared, Wv_shared, Uk, Uv) -> dict:
    """Cache rows of new tokens computed from their inputs X [B, n, d]: for
    every sequence, the shared key and value features and the per-head key and
    value latents of cache_from_inputs (Eqs. (4)-(5)), with the key weights
    W^K_shared, U^K_h and the value weights W^V_shared, U^V_h.  Returns the
    dict append() takes: k_s, v_s [B, n, d_h]; z_k, z_v [B, n, H, r]."""
    X = np.asarray(X, np.float64)
    rows = {"k_s": [], "v_s": [], "z_k": [], "z_v": []}
    for b in range(X.shape[0]):
        k_s, z_k = cache_from_inputs(X[b], Wk_shared, Uk)
        v_s, z_v = cache_from_inputs(X[b], Wv_shared, Uv)
        rows["k_s"].append(k_s)
        rows["v_s"].append(v_s)
        rows["z_k"].append(z_k)
        rows["z_v"].append(z_v)
    return {key: np.stack(val) for key, val in rows.items()}


# ---------------------------------------------------------------------------
# Implied per-head features from the cache.
# Slide "Cache shared features and compact per-head latents":
#   K_h = K_s + R^K_h (B^K_h)^T,   V_h = V_s + R^V_h (B^V_h)^T.
# ---------------------------------------------------------------------------
def implied_kv(k_s, v_s, z_k, z_v, b_k, b_v):
    """k_s, v_s [T, d_h]; z_k, z_v [T, H, r]; b_k, b_v [H, d_h, r]
    -> (K, V), each [H, T, d_h] float64, built explicitly."""
    k_s = np.asarray(k_s, np.float64)
    v_s = np.asarray(v_s, np.float64)
    z_k = np.asarray(z_k, np.float64)
    z_v = np.asarray(z_v, np.float64)
    b_k = np.asarray(b_k, np.float64)
    b_v = np.asarray(b_v, np.float64)
    H = b_k.shape[0]
    K = np.stack([k_s + z_k[:, h, :] @ b_k[h].T for h in range(H)])
    V = np.stack([v_s + z_v[:, h, :] @ b_v[h].T for h in range(H)])
    return K, V


def softmax_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """Textbook single-query attention: a = softmax(scale * K q), o = V^T a.
    q [d_h], K [T, d_h], V [T, d_v].  T == 0 returns zeros (convention)."""
    if K.shape[0] == 0:
        return np.zeros(V.shape[1], np.float64)
    s = (K @ q) * scale
    e = np.exp(s - s.max())
    a = e / e.sum()
    return a @ V


def _default_scale(d_h: int, scale: Optional[float]) -> float:
    # Slide "Compute logits without expanding historical keys": the logits are
    # divided by sqrt(d_h) before the softmax.
    return 1.0 / math.sqrt(d_h) if scale is None or scale <= 0 else float(scale)


def decode(q, k_s, v_s, z_k, z_v, b_k, b_v, seq_lens, scale: Optional[float] = None) -> np.ndarray:
    """One decode step for every sequence and head, plain reconstructed form.

    q [B, H, d_h]; k_s, v_s [B, T, d_h]; z_k, z_v [B, T, H, r]; b_k, b_v [H, d_h, r];
    seq_lens [B].  Returns out [B, H, d_h] float64 where
      out[b, h] = softmax(K_h q_h / sqrt(d_h)) V_h over the first seq_lens[b] tokens
    (slides "Compute logits without expanding historical keys", Eq. (6), and
    "Aggregate values before the residual up-projection", Eq. (7), evaluated
    through the explicitly reconstructed K_h and V_h)."""
    q = np.asarray(q, np.float64)
    B, H, d_h = q.shape
    sc = _default_scale(d_h, scale)
    out = np.zeros((B, H, d_h), np.float64)
    for b in range(B):
        L = int(seq_lens[b])
        if L == 0:
            continue
        K, V = implied_kv(k_s[b, :L], v_s[b, :L], z_k[b, :L], z_v[b, :L], b_k, b_v)
        for h in range(H):
            out[b, h] = softmax_attention(q[b, h], K[h], V[h], sc)
    return out


def prefill(q, k_s, v_s, z_k, z_v, b_k, b_v, scale: Optional[float] = None) -> np.ndarray:
    """Causal attention of L fresh tokens over themselves.

    q [B, L, H, d_h]; k_s, v_s [B, L, d_h]; z_k, z_v [B, L, H, r].
    Query i attends to keys j <= i (0-based), the causal mask of slide
    "Compute logits without expanding historical keys".  Returns [B, L, H, d_h]."""
    q = np.asarray(q, np.float64)
    B, L, H, d_h = q.shape
    sc = _default_scale(d_h, scale)
    out = np.zeros((B, L, H, d_h), np.float64)
    future = np.triu(np.ones((L, L), dtype=bool), k=1)      # j > i
    for b in range(B):
        K, V = implied_kv(k_s[b], v_s[b], z_k[b], z_v[b], b_k, b_v)
        for h in range(H):
            S = (q[b, :, h, :] @ K[h].T) * sc
            S[future] = -np.inf
            E = np.exp(S - S.max(axis=1, keepdims=True))
            A = E / E.sum(axis=1, keepdims=True)
            out[b, :, h, :] = A @ V[h]
    return out


def prefill_with_past(q, k_s, v_s, z_k, z_v, b_k, b_v, start, scale: Optional[float] = None) -> np.ndarray:
    """Causal attention of L new tokens per sequence over everything cached
    before them and over themselves (a prefill chunk, or a decode step of
    several tokens).

    q [B, L, H, d_h].  k_s, v_s [B, T, d_h], z_k, z_v [B, T, H, r] hold the
    cache after the new tokens were written at slots [start[b], start[b] + L).
    New token i of sequence b sits at position start[b] + i and attends to
    the cached tokens j <= start[b] + i: the causal mask of slide "Compute
    logits without expanding historical keys" with start[b] historical keys in
    front.  Returns [B, L, H, d_h]."""
    q = np.asarray(q, np.float64)
    B, L, H, d_h = q.shape
    sc = _default_scale(d_h, scale)
    out = np.zeros((B, L, H, d_h), np.float64)
    for b in range(B):
        s0 = int(start[b])
        n = s0 + L
        K, V = implied_kv(k_s[b, :n], v_s[b, :n], z_k[b, :n], z_v[b, :n], b_k, b_v)
        pos = s0 + np.arange(L)[:, None]                     # absolute position of each new token
        future = np.arange(n)[None, :] > pos                 # keys after the query
        for h in range(H):
            S = (q[b, :, h, :] @ K[h].T) * sc
            S[future] = -np.inf
            E = np.exp(S - S.max(axis=1, keepdims=True))
            A = E / E.sum(axis=1, keepdims=True)
            out[b, :, h, :] = A @ V[h]
    return out


def decode_from_weights(X, q, Wk_shared, Wv_shared, Uk, Uv, Bk, Bv, scale: Optional[float] = None):
    """Decode for one sequence starting from the weights: build W_h explicitly
    (Eqs. (2)-(3)), project every cached input row, K_h = X W^K_h and
    V_h = X W^V_h, then textbook attention.  X [L, d], q [H, d_h] -> [H, d_h]."""
    X = np.asarray(X, np.float64)
    q = np.asarray(q, np.float64)
    H, d_h = q.shape
    sc = _default_scale(d_h, scale)
    WK = head_projections(Wk_shared, Uk, Bk)
    WV = head_projections(Wv_shared, Uv, Bv)
    out = np.zeros((H, d_h), np.float64)
    for h in range(H):
        out[h] = softmax_attention(q[h], X @ WK[h], X @ WV[h], sc)
    return out


def append(cache: dict, pos, new: dict) -> dict:
    """Cache append: the n new tokens of sequence b land in slots
    [pos[b], pos[b] + n) of each of the four cache arrays; every other slot is
    unchanged.  B_h are weights and are not stored (slide "Cache shared
    features and compact per-head latents").  Returns updated copies."""
    outc = {k: np.array(cache[k], copy=True) for k in ("k_s", "v_s", "z_k", "z_v")}
    for key in outc:
        src = new[key]
        n = src.shape[1]
        for b in range(src.shape[0]):
            p = int(pos[b])
            outc[key][b, p:p + n] = src[b]
    return outc


# ---------------------------------------------------------------------------
# Training-side workload.
# Slide "Training learns the base and residuals together" (paper Sec. 3):
# W_shared, U_h and B_h are trained jointly, and training evaluates the full
# per-head K/V.  The forward pass of a layer's attention is the causal
# prefill above; its backward pass is the gradient of a scalar loss with
# respect to every input of that prefill.  Written here the plain way: the
# per-head keys and values are reconstructed explicitly (the "expanded"
# evaluation of the same model), ordinary softmax attention is
# differentiated per head, and the chain rule runs through
#   K_h = K_s + Z^K_h (B^K_h)^T,   V_h = V_s + Z^V_h (B^V_h)^T
# (slide "Cache shared features and compact per-head latents").
# ---------------------------------------------------------------------------
def prefill_forward_lse(q, k_s, v_s, z_k, z_v, b_k, b_v, scale: Optional[float] = None):
    """The causal prefill of ``prefill`` and, for every query row i of every
    head, the natural log-sum-exp of its scaled causal logits,
    lse[b, i, h] = log sum_{j <= i} exp(scale * q_{b,i,h} . k_{h,j}).
    Returns (out [B, L, H, d_h], lse [B, L, H])."""
    q = np.asarray(q, np.float64)
    B, L, H, d_h = q.shape
    sc = _default_scale(d_h, scale)
    out = np.zeros((B, L, H, d_h), np.float64)
    lse = np.zeros((B, L, H), np.float64)
    future = np.triu(np.ones((L, L), dtype=bool), k=1)
    for b in range(B):
        K, V = implied_kv(k_s[b], v_s[b], z_k[b], z_v[b], b_k, b_v)
        for h in range(H):
            S = (q[b, :, h, :] @ K[h].T) * sc
            S[future] = -np.inf
            mx = S.max(axis=1, keepdims=True)
            E = np.exp(S - mx)
            tot = E.sum(axis=1, keepdims=True)
            out[b, :, h, :] = (E / tot) @ V[h]
            lse[b, :, h] = (mx + np.log(tot))[:, 0]
    return out, lse


def prefill_backward(q, k_s, v_s, z_k, z_v, b_k, b_v, d_out, scale: Optional[float] = None) -> dict:
    """Gradients of the scalar sum(d_out * prefill(q, k_s, v_s, z_k, z_v,
    b_k, b_v)) with respect to each input (a vector-Jacobian product).

    Per sequence b and head h, with K_h, V_h reconstructed and the causal
    softmax A = softmax(scale * Q_h K_h^T) (future keys masked):
      dV_h = A^T dO_h,      dA = dO_h V_h^T,
      dS   = A o (dA - rowsum(A o dA))        (derivative of the softmax),
      dQ_h = scale * dS K_h,   dK_h = scale * dS^T Q_h;
    then through K_h = K_s + Z^K_h (B^K_h)^T (and V likewise):
      dK_s = sum_h dK_h,   dZ^K_h = dK_h B^K_h,   dB^K_h = sum_b dK_h^T Z^K_h.
    Returns float64 arrays named after the inputs: dq [B, L, H, d_h],
    dk_s, dv_s [B, L, d_h], dz_k, dz_v [B, L, H, r], db_k, db_v [H, d_h, r]."""
    q = np.asarray(q, np.float64)
    d_out = np.asarray(d_out, np.float64)
    z_k = np.asarray(z_k, np.float64)
    z_v = np.asarray(z_v, np.float64)
    b_k = np.asarray(b_k, np.float64)
    b_v = np.asarray(b_v, np.float64)
    B, L, H, d_h = q.shape
    r = b_k.shape[2]
    sc = _default_scale(d_h, scale)
    g = {"dq": np.zeros_like(q), "dk_s": np.zeros((B, L, d_h)), "dv_s": np.zeros((B, L, d_h)),
         "dz_k": np.zeros((B, L, H, r)), "dz_v": np.zeros((B, L, H, r)),
         "db_k": np.zeros((H, d_h, r)), "db_v": np.zeros((H, d_h, r))}
    future = np.triu(np.ones((L, L), dtype=bool), k=1)
    for b in range(B):
        K, V = implied_kv(k_s[b], v_s[b], z_k[b], z_v[b], b_k, b_v)
        for h in range(H):
            Qh, dO = q[b, :, h, :], d_out[b, :, h, :]
            S = (Qh @ K[h].T) * sc
            S[future] = -np.inf
            E = np.exp(S - S.max(axis=1, keepdims=True))
            A = E / E.sum(axis=1, keepdims=True)
            dV = A.T @ dO
            dA = dO @ V[h].T
            dS = A * (dA - (A * dA).sum(axis=1, keepdims=True))
            g["dq"][b, :, h, :] = sc * (dS @ K[h])
            dK = sc * (dS.T @ Qh)
            g["dk_s"][b] += dK
            g["dv_s"][b] += dV
            g["dz_k"][b, :, h, :] = dK @ b_k[h]
            g["dz_v"][b, :, h, :] = dV @ b_v[h]
            g["db_k"][h] += dK.T @ z_k[b, :, h, :]
            g["db_v"][h] += dV.T @ z_v[b, :, h, :]
    return g
