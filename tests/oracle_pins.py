"""Pins of the float64 oracle against what the pages and mathematics fix.

Each ``pin_*`` takes the oracle module ``O`` and raises AssertionError when
the oracle disagrees with an independent fact: a number printed on the pages
(fixtures under ``tests/golden/``), a closed form, a library routine
(``torch.nn.functional.scaled_dot_product_attention`` in float64 on the CPU),
brute force in pure Python with exactly rounded sums, or an invariant.  None
of them re-types the oracle's own formula.  ``test_oracle_mutations`` runs the
same pins against oracles with planted mistakes and requires each mistake to
be caught.
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
TIGHT = 1e-12


def read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("|")[0].strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def rel_err(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def _rand_cache(seed, B=2, T=37, H=3, d_h=8, r=3, zero_b=False, lens=None):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, d_h))
    k_s = rng.standard_normal((B, T, d_h))
    v_s = rng.standard_normal((B, T, d_h))
    z_k = rng.standard_normal((B, T, H, r))
    z_v = rng.standard_normal((B, T, H, r))
    b_k = rng.standard_normal((H, d_h, r)) / math.sqrt(max(r, 1))
    b_v = rng.standard_normal((H, d_h, r)) / math.sqrt(max(r, 1))
    if zero_b:
        b_k[:] = 0.0
        b_v[:] = 0.0
    seq_lens = np.array(lens if lens is not None else [T] * B, dtype=np.int64)
    return q, k_s, v_s, z_k, z_v, b_k, b_v, seq_lens


def _sdpa(q, K, V, scale, causal=False):
    """Library attention, float64 CPU.  q [..., Lq, d], K/V [..., Lk, d]."""
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(np.ascontiguousarray(q)), torch.from_numpy(np.ascontiguousarray(K)),
        torch.from_numpy(np.ascontiguousarray(V)), is_causal=causal, scale=scale).numpy()


# ---------------------------------------------------------------------------
# Cache accounting against printed numbers.
# ---------------------------------------------------------------------------
def pin_cache_counts_printed(O):
    for mech, H, d_h, r, n_kv, layers, want in read_golden("cache_counts.txt"):
        got = O.cache_elems_per_token(mech, H=int(H), d_h=int(d_h), r=int(r), n_kv=int(n_kv),
                                      layers=int(layers))
        assert got == int(want), (mech, H, d_h, r, n_kv, layers, got, want)


def pin_cache_ratios_printed(O):
    for H, d_h, r, pct, dec in read_golden("cache_ratios.txt"):
        got = 100.0 * O.cache_ratio_vs_mha(int(H), int(d_h), int(r))
        # printed to `dec` decimals, rounded half up
        assert abs(got - float(pct)) <= 0.5 * 10.0 ** (-int(dec)) + 1e-9, (H, d_h, r, got, pct)


def pin_cache_ratio_boxed_form(O):
    # Boxed simplification of Eq. (9): rho = 1/H + r/d_h; r = 0 is MQA (1/H),
    # r = d_h gives 1 + 1/H (slide "The rank directly sets the theoretical cache budget").
    for H in (1, 2, 6, 12, 18, 32, 64):
        for d_h in (16, 64, 128):
            for r in (0, 1, 7, 16, d_h):
                got = Fraction(O.cache_elems_per_token("lrkv", H=H, d_h=d_h, r=r),
                               O.cache_elems_per_token("mha", H=H, d_h=d_h))
                assert got == Fraction(1, H) + Fraction(r, d_h), (H, d_h, r)
                assert abs(O.cache_ratio_vs_mha(H, d_h, r) - float(got)) < 1e-15
            assert O.cache_elems_per_token("lrkv", H=H, d_h=d_h, r=0) == O.cache_elems_per_token("mqa", d_h=d_h)


def pin_table12_megabytes(O):
    for H, r, mb_lrkv, mb_mha in read_golden("table12_megabytes.txt"):
        assert Fraction(O.cache_elems_per_token("lrkv", H=int(H), d_h=128, r=int(r)),
                        O.cache_elems_per_token("mha", H=int(H), d_h=128)) == Fraction(int(mb_lrkv), int(mb_mha))


def pin_kv_param_count_matches_arrays(O):
    # Eq. (10) must equal the number of parameters the weight-level model actually holds.
    for d_h, H, r in ((16, 4, 4), (128, 18, 55), (64, 8, 0)):
        d = H * d_h
        arrays = [np.zeros((d, d_h)), np.zeros((d, d_h)), np.zeros((H, d, r)), np.zeros((H, d, r)),
                  np.zeros((H, d_h, r)), np.zeros((H, d_h, r))]
        assert O.kv_param_count("lrkv", d=d, d_h=d_h, H=H, r=r) == sum(a.size for a in arrays)
        assert O.kv_param_count("mha", d=d, d_h=d_h, H=H) == 2 * H * np.zeros((d, d_h)).size


# ---------------------------------------------------------------------------
# Decode.
# ---------------------------------------------------------------------------
def pin_decode_mqa_reduction(O):
    # B^K = B^V = 0 (and r = 0): every head shares one K/V pair, i.e. MQA
    # (slide "The rank directly sets the theoretical cache budget": r = 0 is MQA-style sharing).
    for r, zero_b in ((3, True), (0, False)):
        q, k_s, v_s, z_k, z_v, b_k, b_v, lens = _rand_cache(11 + r, r=r, zero_b=zero_b, lens=[37, 20])
        got = O.decode(q, k_s, v_s, z_k, z_v, b_k, b_v, lens)
        d_h = q.shape[-1]
        for b in range(q.shape[0]):
            L = int(lens[b])
            K = np.broadcast_to(k_s[b, :L], (q.shape[1], L, d_h))
            V = np.broadcast_to(v_s[b, :L], (q.shape[1], L, d_h))
            want = _sdpa(q[b][:, None, :], K, V, 1.0 / math.sqrt(d_h))[:, 0, :]
            assert rel_err(got[b], want) < TIGHT, (r, b, rel_err(got[b], want))


def pin_decode_mha_special_case(O):
    # r = d_h with B_h = I and a zero shared base makes every head independent:
    # MHA on the latents (slide "The rank directly sets the theoretical cache budget").
    B, T, H, d_h = 2, 29, 4, 8
    q, k_s, v_s, z_k, z_v, _, _, lens = _rand_cache(5, B=B, T=T, H=H, d_h=d_h, r=d_h)
    eye = np.broadcast_to(np.eye(d_h), (H, d_h, d_h)).copy()
    got = O.decode(q, np.zeros_like(k_s), np.zeros_like(v_s), z_k, z_v, eye, eye, lens)
    K = np.transpose(z_k, (0, 2, 1, 3))          # [B, H, T, d_h]
    V = np.transpose(z_v, (0, 2, 1, 3))
    want = _sdpa(q[:, :, None, :], K, V, 1.0 / math.sqrt(d_h))[:, :, 0, :]
    assert rel_err(got, want) < TIGHT


def _absorbed_decode(q, k_s, v_s, z_k, z_v, b_k, b_v, lens):
    """Eqs. (6)-(7) in their absorbed form, written from the slides: project
    the query into r dims, score = q.k_s + (q B^K).z^K, softmax with 1/sqrt(d_h),
    output = a V_s + (a R^V) (B^V)^T.  No K_h or V_h is formed."""
    B, H, d_h = q.shape
    out = np.zeros((B, H, d_h))
    for b in range(B):
        L = int(lens[b])
        for h in range(H):
            qt = q[b, h] @ b_k[h]                                  # q_h B^K_h  (1 x r)
            s = (k_s[b, :L] @ q[b, h] + z_k[b, :L, h, :] @ qt) / math.sqrt(d_h)
            a = np.exp(s - s.max())
            a /= a.sum()
            out[b, h] = a @ v_s[b, :L] + (a @ z_v[b, :L, h, :]) @ b_v[h].T
    return out


def pin_decode_absorbed_equals_reconstructed(O):
    for seed, (B, T, H, d_h, r) in enumerate(((2, 41, 3, 8, 3), (1, 64, 4, 16, 4), (2, 17, 2, 6, 6))):
        lens = [T] + [T - 5] * (B - 1)
        q, k_s, v_s, z_k, z_v, b_k, b_v, lens = _rand_cache(100 + seed, B, T, H, d_h, r, lens=lens)
        got = O.decode(q, k_s, v_s, z_k, z_v, b_k, b_v, lens)
        assert rel_err(got, _absorbed_decode(q, k_s, v_s, z_k, z_v, b_k, b_v, lens)) < TIGHT


def pin_weight_level_equals_cache_level(O):
    # Slide "Training learns the base and residuals together": factored and expanded
    # evaluation of the same LRKV model agree in the linear setting.
    rng = np.random.default_rng(77)
    H, d_h, r, L = 3, 8, 2, 19
    d = H * d_h
    X = rng.standard_normal((L, d))
    Wk, Wv = rng.standard_normal((d, d_h)), rng.standard_normal((d, d_h))
    Uk, Uv = rng.standard_normal((H, d, r)), rng.standard_normal((H, d, r))
    Bk, Bv = rng.standard_normal((H, d_h, r)), rng.standard_normal((H, d_h, r))
    q = rng.standard_normal((H, d_h))
    k_s, z_k = O.cache_from_inputs(X, Wk, Uk)
    v_s, z_v = O.cache_from_inputs(X, Wv, Uv)
    assert rel_err(k_s, X @ Wk) < TIGHT and rel_err(z_k[:, 1, :], X @ Uk[1]) < TIGHT
    cache_level = O.decode(q[None], k_s[None], v_s[None], z_k[None], z_v[None], Bk, Bv, [L])[0]
    weight_level = O.decode_from_weights(X, q, Wk, Wv, Uk, Uv, Bk, Bv)
    assert rel_err(cache_level, weight_level) < TIGHT


def pin_weight_level_on_tiny_workload(O, inputs):
    # The tiny workload has d = H * d_h = T = 64, so X = I_64 with W_shared := K_s and
    # U_h := R_h reproduces exactly its cache; decoding from the weights must match.
    q, k_s, v_s, z_k, z_v, b_k, b_v, lens = inputs
    T = k_s.shape[1]
    H, d_h = q.shape[1], q.shape[2]
    assert H * d_h == T
    X = np.eye(T)
    Uk = np.transpose(z_k[0], (1, 0, 2))    # [H, d=T, r]
    Uv = np.transpose(z_v[0], (1, 0, 2))
    weight_level = O.decode_from_weights(X, q[0], k_s[0], v_s[0], Uk, Uv, b_k, b_v)
    cache_level = O.decode(q, k_s, v_s, z_k, z_v, b_k, b_v, lens)[0]
    assert rel_err(cache_level, weight_level) < TIGHT


def brute_force_decode(q, k_s, v_s, z_k, z_v, b_k, b_v, lens):
    """Pure-Python loops with exactly rounded sums (math.fsum): the implied
    key/value of every (head, token) element by element, then the softmax."""
    B, H, d_h = q.shape
    r = z_k.shape[-1]
    out = np.zeros((B, H, d_h))
    for b in range(B):
        L = int(lens[b])
        for h in range(H):
            scores = []
            vals = []
            for t in range(L):
                key = [k_s[b, t, i] + math.fsum(b_k[h, i, j] * z_k[b, t, h, j] for j in range(r))
                       for i in range(d_h)]
                val = [v_s[b, t, i] + math.fsum(b_v[h, i, j] * z_v[b, t, h, j] for j in range(r))
                       for i in range(d_h)]
                scores.append(math.fsum(q[b, h, i] * key[i] for i in range(d_h)) / math.sqrt(d_h))
                vals.append(val)
            if L == 0:
                continue
            m = max(scores)
            w = [math.exp(s - m) for s in scores]
            z = math.fsum(w)
            for i in range(d_h):
                out[b, h, i] = math.fsum(w[t] * vals[t][i] for t in range(L)) / z
    return out


def pin_decode_brute_force(O, inputs):
    got = O.decode(*inputs)
    assert rel_err(got, brute_force_decode(*inputs)) < 1e-13


def pin_decode_closed_forms(O):
    # One cached token: the softmax weight is 1, so o_h = v_s + B^V_h z^V_h.
    q, k_s, v_s, z_k, z_v, b_k, b_v, _ = _rand_cache(21, B=2, T=5, H=3, d_h=6, r=2)
    got = O.decode(q, k_s, v_s, z_k, z_v, b_k, b_v, [1, 1])
    for b in range(2):
        for h in range(3):
            want = v_s[b, 0] + np.einsum("ij,j->i", b_v[h], z_v[b, 0, h])
            assert rel_err(got[b, h], want) < TIGHT
    # Zero query: uniform weights, so o_h = mean_t v_s + B^V_h mean_t z^V_h.
    got = O.decode(np.zeros_like(q), k_s, v_s, z_k, z_v, b_k, b_v, [5, 3])
    for b, L in ((0, 5), (1, 3)):
        for h in range(3):
            want = v_s[b, :L].mean(0) + np.einsum("ij,j->i", b_v[h], z_v[b, :L, h].mean(0))
            assert rel_err(got[b, h], want) < TIGHT
    # Empty sequence: all-zero output (convention).
    got = O.decode(q, k_s, v_s, z_k, z_v, b_k, b_v, [0, 2])
    assert np.all(got[0] == 0.0) and np.any(got[1] != 0.0)


def pin_decode_invariances(O):
    q, k_s, v_s, z_k, z_v, b_k, b_v, lens = _rand_cache(31, B=1, T=23, H=3, d_h=8, r=3)
    base = O.decode(q, k_s, v_s, z_k, z_v, b_k, b_v, lens)
    # No positions: permuting the cached tokens leaves the output unchanged.
    perm = np.random.default_rng(0).permutation(23)
    got = O.decode(q, k_s[:, perm], v_s[:, perm], z_k[:, perm], z_v[:, perm], b_k, b_v, lens)
    assert rel_err(got, base) < TIGHT
    # Shifting every shared key by one vector u moves all scores of a head by the
    # same constant q_h.u/sqrt(d_h); softmax is unchanged by that.
    u = np.random.default_rng(1).standard_normal(8) * 3.0
    got = O.decode(q, k_s + u, v_s, z_k, z_v, b_k, b_v, lens)
    assert rel_err(got, base) < TIGHT
    # Scaling the query by c is the same as scaling the softmax scale by c.
    got = O.decode(0.5 * q, k_s, v_s, z_k, z_v, b_k, b_v, lens)
    want = O.decode(q, k_s, v_s, z_k, z_v, b_k, b_v, lens, scale=0.5 / math.sqrt(8))
    assert rel_err(got, want) < TIGHT
    # Tokens beyond the length are ignored, whatever they hold.
    k2 = k_s.copy()
    k2[:, 20:] = 1e3
    got = O.decode(q, k2, v_s, z_k, z_v, b_k, b_v, [20])
    want = O.decode(q, k_s[:, :20], v_s[:, :20], z_k[:, :20], z_v[:, :20], b_k, b_v, [20])
    assert rel_err(got, want) < TIGHT


# ---------------------------------------------------------------------------
# Prefill.
# ---------------------------------------------------------------------------
def _rand_prefill(seed, B=2, L=13, H=3, d_h=8, r=3, zero_b=False):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, L, H, d_h))
    k_s = rng.standard_normal((B, L, d_h))
    v_s = rng.standard_normal((B, L, d_h))
    z_k = rng.standard_normal((B, L, H, r))
    z_v = rng.standard_normal((B, L, H, r))
    b_k = rng.standard_normal((H, d_h, r)) / math.sqrt(max(r, 1))
    b_v = rng.standard_normal((H, d_h, r)) / math.sqrt(max(r, 1))
    if zero_b:
        b_k[:] = 0
        b_v[:] = 0
    return q, k_s, v_s, z_k, z_v, b_k, b_v


def pin_prefill_mqa_causal_sdpa(O):
    q, k_s, v_s, z_k, z_v, b_k, b_v = _rand_prefill(41, zero_b=True)
    got = O.prefill(q, k_s, v_s, z_k, z_v, b_k, b_v)
    B, L, H, d_h = q.shape
    qh = np.transpose(q, (0, 2, 1, 3))                      # [B, H, L, d_h]
    K = np.broadcast_to(k_s[:, None], (B, H, L, d_h))
    V = np.broadcast_to(v_s[:, None], (B, H, L, d_h))
    want = np.transpose(_sdpa(qh, K, V, 1.0 / math.sqrt(d_h), causal=True), (0, 2, 1, 3))
    assert rel_err(got, want) < TIGHT


def pin_prefill_mha_causal_sdpa(O):
    B, L, H, d_h = 1, 11, 2, 4
    q, k_s, v_s, z_k, z_v, _, _ = _rand_prefill(43, B, L, H, d_h, r=d_h)
    eye = np.broadcast_to(np.eye(d_h), (H, d_h, d_h)).copy()
    got = O.prefill(q, 0 * k_s, 0 * v_s, z_k, z_v, eye, eye)
    want = _sdpa(np.transpose(q, (0, 2, 1, 3)), np.transpose(z_k, (0, 2, 1, 3)),
                 np.transpose(z_v, (0, 2, 1, 3)), 1.0 / math.sqrt(d_h), causal=True)
    assert rel_err(got, np.transpose(want, (0, 2, 1, 3))) < TIGHT


def pin_prefill_rows_are_decodes(O):
    # Row i of causal prefill is a decode of query i over the first i+1 tokens,
    # which in turn is pinned above; row 0 sees only token 0.
    q, k_s, v_s, z_k, z_v, b_k, b_v = _rand_prefill(47)
    got = O.prefill(q, k_s, v_s, z_k, z_v, b_k, b_v)
    B, L = q.shape[:2]
    for i in (0, 1, 6, L - 1):
        want = _absorbed_decode(q[:, i], k_s, v_s, z_k, z_v, b_k, b_v, [i + 1] * B)
        assert rel_err(got[:, i], want) < TIGHT, i
    for b in range(B):
        for h in range(q.shape[2]):
            assert rel_err(got[b, 0, h], v_s[b, 0] + b_v[h] @ z_v[b, 0, h]) < TIGHT


# ---------------------------------------------------------------------------
# Append.
# ---------------------------------------------------------------------------
def _rand_past(seed, B=3, L=9, T=40, H=3, d_h=8, r=3, zero_b=False):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, L, H, d_h))
    k_s, v_s = rng.standard_normal((B, T, d_h)), rng.standard_normal((B, T, d_h))
    z_k, z_v = rng.standard_normal((B, T, H, r)), rng.standard_normal((B, T, H, r))
    b_k = rng.standard_normal((H, d_h, r)) / math.sqrt(r)
    b_v = rng.standard_normal((H, d_h, r)) / math.sqrt(r)
    if zero_b:
        b_k[:] = 0.0
        b_v[:] = 0.0
    start = np.array([0, 17, T - L][:B], dtype=np.int64)
    return q, k_s, v_s, z_k, z_v, b_k, b_v, start


def pin_prefill_with_past_rows_are_decodes(O):
    # New token i of a chunk is a decode of its query over the first
    # start + i + 1 cached tokens (decode itself is pinned to a library
    # routine and to brute force).
    q, k_s, v_s, z_k, z_v, b_k, b_v, start = _rand_past(61)
    got = O.prefill_with_past(q, k_s, v_s, z_k, z_v, b_k, b_v, start)
    B, L = q.shape[:2]
    for b in range(B):
        for i in range(L):
            want = O.decode(q[b:b + 1, i], k_s[b:b + 1], v_s[b:b + 1], z_k[b:b + 1], z_v[b:b + 1], b_k, b_v,
                            [int(start[b]) + i + 1])
            assert rel_err(got[b, i], want[0]) < TIGHT, (b, i)


def pin_prefill_with_past_mqa_sdpa(O):
    # B = 0: every head attends to K_s/V_s under the shifted causal mask;
    # torch's attention with an explicit boolean mask is the reference.
    q, k_s, v_s, z_k, z_v, b_k, b_v, start = _rand_past(67, zero_b=True)
    got = O.prefill_with_past(q, k_s, v_s, z_k, z_v, b_k, b_v, start)
    B, L, H, d_h = q.shape
    for b in range(B):
        n = int(start[b]) + L
        allowed = np.arange(n)[None, :] <= (int(start[b]) + np.arange(L))[:, None]
        qh = torch.from_numpy(np.ascontiguousarray(q[b].transpose(1, 0, 2)))
        Kb = torch.from_numpy(np.ascontiguousarray(np.broadcast_to(k_s[b, :n], (H, n, d_h))))
        Vb = torch.from_numpy(np.ascontiguousarray(np.broadcast_to(v_s[b, :n], (H, n, d_h))))
        ref = torch.nn.functional.scaled_dot_product_attention(
            qh, Kb, Vb, attn_mask=torch.from_numpy(allowed), scale=1.0 / math.sqrt(d_h)).numpy()
        assert rel_err(got[b], ref.transpose(1, 0, 2)) < TIGHT, b


def pin_chunked_prefill_equals_full(O):
    # Processing a sequence in chunks, each over everything before it, gives
    # the rows of one causal prefill over the whole sequence.
    rng = np.random.default_rng(71)
    B, T, H, d_h, r = 2, 23, 2, 8, 3
    q = rng.standard_normal((B, T, H, d_h))
    k_s, v_s = rng.standard_normal((B, T, d_h)), rng.standard_normal((B, T, d_h))
    z_k, z_v = rng.standard_normal((B, T, H, r)), rng.standard_normal((B, T, H, r))
    b_k, b_v = rng.standard_normal((H, d_h, r)) / 2, rng.standard_normal((H, d_h, r)) / 2
    full = O.prefill(q, k_s, v_s, z_k, z_v, b_k, b_v)
    for lo, hi in ((0, 8), (8, 9), (9, 23)):
        part = O.prefill_with_past(q[:, lo:hi], k_s, v_s, z_k, z_v, b_k, b_v, np.full(B, lo))
        assert rel_err(part, full[:, lo:hi]) < TIGHT, (lo, hi)


def pin_append_slots(O):
    rng = np.random.default_rng(3)
    B, T, H, d_h, r, n = 3, 16, 2, 4, 2, 5
    cache = dict(k_s=rng.standard_normal((B, T, d_h)), v_s=rng.standard_normal((B, T, d_h)),
                 z_k=rng.standard_normal((B, T, H, r)), z_v=rng.standard_normal((B, T, H, r)))
    new = dict(k_s=rng.standard_normal((B, n, d_h)), v_s=rng.standard_normal((B, n, d_h)),
               z_k=rng.standard_normal((B, n, H, r)), z_v=rng.standard_normal((B, n, H, r)))
    pos = [0, 7, T - n]
    got = O.append(cache, pos, new)
    for key in cache:
        for b in range(B):
            for t in range(T):
                if pos[b] <= t < pos[b] + n:
                    assert np.array_equal(got[key][b, t], new[key][b, t - pos[b]])
                else:
                    assert np.array_equal(got[key][b, t], cache[key][b, t])
    # cache size per token is exactly the element count of the four rows
    per_tok = sum(int(np.prod(got[k].shape[2:])) for k in got)
    assert per_tok == O.cache_elems_per_token("lrkv", H=H, d_h=d_h, r=r)


def _rand_projection(seed, d=5, H=2, d_h=4, r=2):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((d, d_h)), rng.standard_normal((d, d_h)),
            rng.standard_normal((H, d, r)), rng.standard_normal((H, d, r)))


def pin_projected_rows_brute_force(O):
    # Every cached element of a new token is one exactly rounded dot product of
    # its input row with one weight column (slide "Cache shared features and
    # compact per-head latents", Eqs. (4)-(5)), in the cache's [B, n, H, r] order.
    rng = np.random.default_rng(11)
    B, n, d, H, d_h, r = 2, 3, 5, 2, 4, 3
    Wk, Wv, Uk, Uv = _rand_projection(12, d, H, d_h, r)
    X = rng.standard_normal((B, n, d))
    got = O.projected_rows(X, Wk, Wv, Uk, Uv)
    for b in range(B):
        for i in range(n):
            x = X[b, i]
            for c in range(d_h):
                assert abs(got["k_s"][b, i, c] - math.fsum(x[k] * Wk[k, c] for k in range(d))) < 1e-13
                assert abs(got["v_s"][b, i, c] - math.fsum(x[k] * Wv[k, c] for k in range(d))) < 1e-13
            for h in range(H):
                for j in range(r):
                    assert abs(got["z_k"][b, i, h, j] - math.fsum(x[k] * Uk[h, k, j] for k in range(d))) < 1e-13
                    assert abs(got["z_v"][b, i, h, j] - math.fsum(x[k] * Uv[h, k, j] for k in range(d))) < 1e-13


def pin_projected_rows_identity_inputs(O):
    # Unit input rows pick out weight rows: X = I_d gives back W_shared and,
    # for head h, U_h (as [d, H, r] in the cache's latent order).
    d, H, d_h, r = 6, 3, 4, 2
    Wk, Wv, Uk, Uv = _rand_projection(13, d, H, d_h, r)
    got = O.projected_rows(np.eye(d)[None], Wk, Wv, Uk, Uv)
    assert np.array_equal(got["k_s"][0], Wk) and np.array_equal(got["v_s"][0], Wv)
    assert np.array_equal(got["z_k"][0], np.transpose(Uk, (1, 0, 2)))
    assert np.array_equal(got["z_v"][0], np.transpose(Uv, (1, 0, 2)))


def pin_projected_rows_decode_like_weights(O):
    # Rows projected from inputs, decoded from the cache, equal attention with
    # the explicit per-head projections W_h = W_shared + U_h B_h^T (Eqs. (2)-(5)).
    rng = np.random.default_rng(14)
    d, H, d_h, r, L = 7, 2, 4, 3, 9
    Wk, Wv, Uk, Uv = _rand_projection(15, d, H, d_h, r)
    Bk, Bv = rng.standard_normal((H, d_h, r)), rng.standard_normal((H, d_h, r))
    X = rng.standard_normal((1, L, d))
    q = rng.standard_normal((H, d_h))
    rows = O.projected_rows(X, Wk, Wv, Uk, Uv)
    got = O.decode(q[None], rows["k_s"], rows["v_s"], rows["z_k"], rows["z_v"], Bk, Bv, [L])[0]
    WK = np.stack([Wk + Uk[h] @ Bk[h].T for h in range(H)])
    WV = np.stack([Wv + Uv[h] @ Bv[h].T for h in range(H)])
    ref = np.stack([_sdpa(q[h][None], X[0] @ WK[h], X[0] @ WV[h], 1.0 / math.sqrt(d_h))[0] for h in range(H)])
    assert rel_err(got, ref) < 1e-12


# ---------------------------------------------------------------------------
# Training-side forward (log-sum-exp) and backward (slide "Training learns
# the base and residuals together").
# ---------------------------------------------------------------------------
_GRAD_NAMES = ("dq", "dk_s", "dv_s", "dz_k", "dz_v", "db_k", "db_v")


def pin_forward_lse_brute_force(O):
    # lse[b, i, h] = log sum_{j <= i} exp(scale q.k_{h,j}), with every logit
    # built by scalar loops (math.fsum) straight from the cache definition
    # k_{h,j} = k_{s,j} + B^K_h z^K_{j,h}, and the log-sum-exp from scipy
    from scipy.special import logsumexp
    q, k_s, v_s, z_k, z_v, b_k, b_v = _rand_prefill(53, B=1, L=5, H=2, d_h=3, r=2)
    out, lse = O.prefill_forward_lse(q, k_s, v_s, z_k, z_v, b_k, b_v)
    assert rel_err(out, O.prefill(q, k_s, v_s, z_k, z_v, b_k, b_v)) < TIGHT
    B, L, H, d_h = q.shape
    r = b_k.shape[2]
    sc = 1.0 / math.sqrt(d_h)
    for b in range(B):
        for h in range(H):
            for i in range(L):
                logits = []
                for j in range(i + 1):
                    kj = [k_s[b, j, e] + math.fsum(b_k[h, e, c] * z_k[b, j, h, c] for c in range(r))
                          for e in range(d_h)]
                    logits.append(sc * math.fsum(q[b, i, h, e] * kj[e] for e in range(d_h)))
                assert abs(lse[b, i, h] - logsumexp(logits)) < 1e-12 * max(1.0, abs(lse[b, i, h]))


def _loss(O, args, d_out):
    return float(np.sum(d_out * O.prefill(*args)))


def pin_backward_finite_differences(O):
    # Every gradient element against a central difference of the (pinned)
    # forward oracle: sum(d_out * prefill(x)) at x +- eps e_k.
    rng = np.random.default_rng(59)
    args = list(_rand_prefill(59, B=2, L=4, H=2, d_h=3, r=2))
    d_out = rng.standard_normal(args[0].shape)
    g = O.prefill_backward(*args, d_out)
    eps = 1e-6
    for idx, name in enumerate(_GRAD_NAMES):
        x = args[idx]
        fd = np.zeros_like(x)
        for k in np.ndindex(x.shape):
            old = x[k]
            x[k] = old + eps
            up = _loss(O, args, d_out)
            x[k] = old - eps
            dn = _loss(O, args, d_out)
            x[k] = old
            fd[k] = (up - dn) / (2 * eps)
        err = float(np.max(np.abs(g[name] - fd)) / max(np.max(np.abs(fd)), 1e-30))
        assert err < 1e-6, (name, err)


def pin_backward_torch_autograd(O):
    # The same gradients by torch autograd (float64, CPU) through the library
    # attention routine on K_h = K_s + Z^K_h B^K_h^T and V_h likewise.
    rng = np.random.default_rng(61)
    args = _rand_prefill(61, B=2, L=9, H=3, d_h=4, r=3)
    d_out = rng.standard_normal(args[0].shape)
    g = O.prefill_backward(*args, d_out)
    t = [torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in args]
    q, k_s, v_s, z_k, z_v, b_k, b_v = t
    K = k_s[:, None] + torch.einsum("blhr,hdr->bhld", z_k, b_k)       # [B, H, L, d_h]
    V = v_s[:, None] + torch.einsum("blhr,hdr->bhld", z_v, b_v)
    out = torch.nn.functional.scaled_dot_product_attention(q.permute(0, 2, 1, 3), K, V, is_causal=True,
                                                           scale=1.0 / math.sqrt(q.shape[-1]))
    (out.permute(0, 2, 1, 3) * torch.from_numpy(d_out)).sum().backward()
    for name, x in zip(_GRAD_NAMES, t):
        assert rel_err(g[name], x.grad.numpy()) < TIGHT, name


def pin_backward_mqa_sdpa(O):
    # B^K = B^V = 0: LRKV is MQA, and the shared rows get the heads' summed
    # key/value gradients of the library routine; the latents get none.
    rng = np.random.default_rng(67)
    q, k_s, v_s, z_k, z_v, b_k, b_v = _rand_prefill(67, B=1, L=7, H=3, d_h=4, r=2, zero_b=True)
    d_out = rng.standard_normal(q.shape)
    g = O.prefill_backward(q, k_s, v_s, z_k, z_v, b_k, b_v, d_out)
    B, L, H, d_h = q.shape
    tq = torch.tensor(np.transpose(q, (0, 2, 1, 3)).copy(), requires_grad=True)
    tk = torch.tensor(np.broadcast_to(k_s[:, None], (B, H, L, d_h)).copy(), requires_grad=True)
    tv = torch.tensor(np.broadcast_to(v_s[:, None], (B, H, L, d_h)).copy(), requires_grad=True)
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=1.0 / math.sqrt(d_h))
    (out * torch.from_numpy(np.transpose(d_out, (0, 2, 1, 3)).copy())).sum().backward()
    assert rel_err(g["dq"], np.transpose(tq.grad.numpy(), (0, 2, 1, 3))) < TIGHT
    assert rel_err(g["dk_s"], tk.grad.numpy().sum(axis=1)) < TIGHT
    assert rel_err(g["dv_s"], tv.grad.numpy().sum(axis=1)) < TIGHT
    assert np.all(g["dz_k"] == 0) and np.all(g["dz_v"] == 0)
    # dB^K_h = dK_h^T Z^K_h with the library's per-head key gradient
    dk_h = np.transpose(tk.grad.numpy(), (0, 2, 1, 3))                 # [B, L, H, d_h]
    want = np.einsum("blhd,blhr->hdr", dk_h, z_k)
    assert rel_err(g["db_k"], want) < TIGHT


def pin_backward_single_token(O):
    # L = 1: the softmax over one key is constant, so nothing upstream of the
    # logits gets a gradient; the value path is linear.
    rng = np.random.default_rng(71)
    q, k_s, v_s, z_k, z_v, b_k, b_v = _rand_prefill(71, B=2, L=1, H=3, d_h=4, r=2)
    d_out = rng.standard_normal(q.shape)
    g = O.prefill_backward(q, k_s, v_s, z_k, z_v, b_k, b_v, d_out)
    for name in ("dq", "dk_s", "dz_k", "db_k"):
        assert np.max(np.abs(g[name])) < 1e-14, name
    assert rel_err(g["dv_s"], d_out.sum(axis=2)) < TIGHT
    assert rel_err(g["dz_v"], np.einsum("blhd,hdr->blhr", d_out, b_v)) < TIGHT
    assert rel_err(g["db_v"], np.einsum("blhd,blhr->hdr", d_out, z_v)) < TIGHT


ALL_PINS = [
    pin_cache_counts_printed, pin_cache_ratios_printed, pin_cache_ratio_boxed_form,
    pin_table12_megabytes, pin_kv_param_count_matches_arrays, pin_decode_mqa_reduction,
    pin_decode_mha_special_case, pin_decode_absorbed_equals_reconstructed,
    pin_weight_level_equals_cache_level, pin_decode_closed_forms, pin_decode_invariances,
    pin_prefill_mqa_causal_sdpa, pin_prefill_mha_causal_sdpa, pin_prefill_rows_are_decodes,
    pin_prefill_with_past_rows_are_decodes, pin_prefill_with_past_mqa_sdpa, pin_chunked_prefill_equals_full,
    pin_append_slots, pin_projected_rows_brute_force, pin_projected_rows_identity_inputs,
    pin_projected_rows_decode_like_weights, pin_forward_lse_brute_force, pin_backward_finite_differences,
    pin_backward_torch_autograd, pin_backward_mqa_sdpa, pin_backward_single_token,
]
