"""Seeded synthetic workloads for LRKV compressed-cache attention.

This module draws inputs and nothing else: it holds none of the method's
arithmetic, so the float64 oracle and the HIP path can both be fed from it
without sharing any computation.  Every array is produced on the host with
``numpy.random.default_rng(seed)``; bf16 workloads are drawn in float32 and
rounded once to bfloat16 (round to nearest, ties to even), so both sides see
the identical rounded values (the oracle upcasts them exactly).

Value distributions follow the LRKV cache definition (Low-Rank Key Value
Attention, slide "Cache shared features and compact per-head latents",
Eqs. (4)-(5)): queries, shared bases K_s/V_s and per-head latents R_h are
N(0, 1); the per-head factors B_h are N(0, 1/r) (variance 1/r), so that
B_h z has unit variance per element, like the base.

Draw order (fixed, part of the workload definition):
  decode : lengths (ragged workloads only), q, then per sequence b in order
           K_s[b,:len], V_s[b,:len], Z^K[b,:len], Z^V[b,:len]; then B^K, B^V.
  prefill: Q, K_s, V_s, Z^K, Z^V, B^K, B^V.
  projection: X, W^K_shared, W^V_shared, U^K, U^V.
Cache slots at or beyond a sequence's length are zero.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

__all__ = [
    "DecodeWorkload", "PrefillWorkload", "DECODE_WORKLOADS", "PREFILL_WORKLOADS",
    "f32_to_bf16_bits", "bf16_bits_to_f32", "decode_inputs", "prefill_inputs",
    "append_inputs", "as_f64", "projection_inputs", "mha_inputs", "train_inputs",
]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def as_f64(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 view of a stored array (float32 values, or bf16 bit patterns)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(arr).astype(np.float64)
    return np.asarray(arr, dtype=np.float64)


@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    name: str
    batch: int
    heads: int
    head_dim: int
    rank: int
    capacity: int                 # cache slots per sequence (row stride)
    dtype: str                    # "f32" or "bf16"
    seed: int
    ragged: Optional[tuple] = None   # (lo, hi) inclusive length range, else every length == capacity


@dataclasses.dataclass(frozen=True)
class PrefillWorkload:
    name: str
    batch: int
    seq_len: int
    heads: int
    head_dim: int
    rank: int
    dtype: str
    seed: int


DECODE_WORKLOADS = {
    w.name: w for w in [
        DecodeWorkload("tiny_f32_T64", 1, 4, 16, 4, 64, "f32", 20261202),
        DecodeWorkload("small_bf16_T2k", 8, 8, 64, 8, 2048, "bf16", 20261203),
        DecodeWorkload("mid_bf16_T8k", 32, 32, 128, 16, 8192, "bf16", 20261204),
        DecodeWorkload("ragged_bf16_T1k_64k", 16, 32, 128, 32, 65536, "bf16", 20261205,
                       ragged=(1024, 65536)),
        # a rank the pages train: the largest model of Table 7 (32 heads of
        # width 128, rank 54) at 8K context; the any-rank scan takes it
        DecodeWorkload("rank54_bf16_T8k", 16, 32, 128, 54, 8192, "bf16", 20261209),
    ]
}

PREFILL_WORKLOADS = {
    w.name: w for w in [
        PrefillWorkload("prefill_bf16_L4k", 4, 4096, 32, 128, 16, "bf16", 20261206),
        # one sequence of the same length at trained ranks (the windowed
        # MFMA prefill): the 2.5B configuration (32 heads, rank 54), an odd
        # rank (18 heads, rank 55) and the top of the rank sweep (16 heads,
        # rank 128); and an odd number of heads at an odd rank (9 heads,
        # rank 55: the vector-ALU prefill)
        PrefillWorkload("prefill_bf16_L4k_r54", 1, 4096, 32, 128, 54, "bf16", 20261210),
        PrefillWorkload("prefill_bf16_L4k_r55", 1, 4096, 18, 128, 55, "bf16", 20261211),
        PrefillWorkload("prefill_bf16_L4k_r128", 1, 4096, 16, 128, 128, "bf16", 20261212),
        PrefillWorkload("prefill_bf16_L4k_h9_r55", 1, 4096, 9, 128, 55, "bf16", 20261213),
    ]
}


def _store(x32: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x32) if dtype == "bf16" else np.ascontiguousarray(x32, dtype=np.float32)


def _b_factor(rng, H, d_h, r):
    b = rng.standard_normal((H, d_h, r), dtype=np.float32)
    if r > 0:
        b *= np.float32(1.0 / np.sqrt(r))
    return b


def decode_inputs(wl: DecodeWorkload, *, batch: Optional[int] = None, seed: Optional[int] = None,
                  capacity: Optional[int] = None, lens: Optional[np.ndarray] = None) -> dict:
    """Draw one decode workload.  ``batch``/``capacity``/``lens``/``seed`` override the
    workload's values (used for reduced-size parity cases of the same distribution)."""
    B = wl.batch if batch is None else batch
    T = wl.capacity if capacity is None else capacity
    H, d_h, r, dt = wl.heads, wl.head_dim, wl.rank, wl.dtype
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    if lens is not None:
        seq_lens = np.asarray(lens, dtype=np.int32)
    elif wl.ragged is not None:
        lo, hi = wl.ragged
        seq_lens = rng.integers(min(lo, T), min(hi, T), size=B, endpoint=True).astype(np.int32)
    else:
        seq_lens = np.full(B, T, dtype=np.int32)
    assert seq_lens.shape == (B,) and int(seq_lens.max(initial=0)) <= T
    q = rng.standard_normal((B, H, d_h), dtype=np.float32)
    sdt = np.uint16 if dt == "bf16" else np.float32
    k_s = np.zeros((B, T, d_h), sdt)
    v_s = np.zeros((B, T, d_h), sdt)
    z_k = np.zeros((B, T, H, r), sdt)
    z_v = np.zeros((B, T, H, r), sdt)
    for b in range(B):
        L = int(seq_lens[b])
        k_s[b, :L] = _store(rng.standard_normal((L, d_h), dtype=np.float32), dt)
        v_s[b, :L] = _store(rng.standard_normal((L, d_h), dtype=np.float32), dt)
        z_k[b, :L] = _store(rng.standard_normal((L, H, r), dtype=np.float32), dt)
        z_v[b, :L] = _store(rng.standard_normal((L, H, r), dtype=np.float32), dt)
    b_k = _b_factor(rng, H, d_h, r)
    b_v = _b_factor(rng, H, d_h, r)
    return dict(q=_store(q, dt), k_s=k_s, v_s=v_s, z_k=z_k, z_v=z_v,
                b_k=_store(b_k, dt), b_v=_store(b_v, dt), seq_lens=seq_lens,
                dtype=dt, heads=H, head_dim=d_h, rank=r, capacity=T)


def prefill_inputs(wl: PrefillWorkload, *, batch: Optional[int] = None, seq_len: Optional[int] = None,
                   seed: Optional[int] = None) -> dict:
    B = wl.batch if batch is None else batch
    L = wl.seq_len if seq_len is None else seq_len
    H, d_h, r, dt = wl.heads, wl.head_dim, wl.rank, wl.dtype
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    q = rng.standard_normal((B, L, H, d_h), dtype=np.float32)
    k_s = rng.standard_normal((B, L, d_h), dtype=np.float32)
    v_s = rng.standard_normal((B, L, d_h), dtype=np.float32)
    z_k = rng.standard_normal((B, L, H, r), dtype=np.float32)
    z_v = rng.standard_normal((B, L, H, r), dtype=np.float32)
    b_k = _b_factor(rng, H, d_h, r)
    b_v = _b_factor(rng, H, d_h, r)
    return dict(q=_store(q, dt), k_s=_store(k_s, dt), v_s=_store(v_s, dt), z_k=_store(z_k, dt),
                z_v=_store(z_v, dt), b_k=_store(b_k, dt), b_v=_store(b_v, dt),
                dtype=dt, heads=H, head_dim=d_h, rank=r, seq_len=L)


def train_inputs(wl: PrefillWorkload, *, batch: Optional[int] = None, seq_len: Optional[int] = None,
                 seed: Optional[int] = None) -> dict:
    """A prefill workload plus the upstream gradient of its output for a
    training step: d_out [B, L, H, d_h] ~ N(0, 1), drawn from a stream of its
    own (seed, 1) so that the forward inputs equal ``prefill_inputs``'s."""
    d = prefill_inputs(wl, batch=batch, seq_len=seq_len, seed=seed)
    B, L = d["q"].shape[0], d["q"].shape[1]
    rng = np.random.default_rng([wl.seed if seed is None else seed, 1])
    d_out = rng.standard_normal((B, L, wl.heads, wl.head_dim), dtype=np.float32)
    d["d_out"] = _store(d_out, wl.dtype)
    return d


def append_inputs(B: int, n: int, H: int, d_h: int, r: int, dtype: str, seed: int) -> dict:
    """New-token rows for a cache append: K_s/V_s rows [B,n,d_h], latents [B,n,H,r]."""
    rng = np.random.default_rng(seed)
    k_s = rng.standard_normal((B, n, d_h), dtype=np.float32)
    v_s = rng.standard_normal((B, n, d_h), dtype=np.float32)
    z_k = rng.standard_normal((B, n, H, r), dtype=np.float32)
    z_v = rng.standard_normal((B, n, H, r), dtype=np.float32)
    return dict(k_s=_store(k_s, dtype), v_s=_store(v_s, dtype), z_k=_store(z_k, dtype),
                z_v=_store(z_v, dtype), dtype=dtype)


SENTINEL = 30.0      # cache slots outside a sequence's history: never to be read as keys


def chunk_inputs(*, batch: int, heads: int, head_dim: int, rank: int, capacity: int, starts, n_new: int,
                 seed: int, dtype: str = "bf16") -> dict:
    """A cache with starts[b] tokens of history per sequence (N(0,1) rows and
    latents; every other slot holds SENTINEL) and n_new new tokens per
    sequence drawn like a prefill workload (q, rows, latents N(0,1),
    B ~ N(0, 1/r)).  Returns the history cache under ``cache_*`` and the new
    tokens, queries and weights under the prefill names."""
    starts = np.asarray(starts, dtype=np.int32)
    assert starts.shape == (batch,) and int(starts.max(initial=0)) + n_new <= capacity
    rng = np.random.default_rng(seed)
    B, H, d_h, r, T = batch, heads, head_dim, rank, capacity
    cache = {
        "cache_k_s": np.full((B, T, d_h), SENTINEL, np.float32),
        "cache_v_s": np.full((B, T, d_h), SENTINEL, np.float32),
        "cache_z_k": np.full((B, T, H, r), SENTINEL, np.float32),
        "cache_z_v": np.full((B, T, H, r), SENTINEL, np.float32),
    }
    for b in range(B):
        s0 = int(starts[b])
        cache["cache_k_s"][b, :s0] = rng.standard_normal((s0, d_h), dtype=np.float32)
        cache["cache_v_s"][b, :s0] = rng.standard_normal((s0, d_h), dtype=np.float32)
        cache["cache_z_k"][b, :s0] = rng.standard_normal((s0, H, r), dtype=np.float32)
        cache["cache_z_v"][b, :s0] = rng.standard_normal((s0, H, r), dtype=np.float32)
    new = prefill_inputs(PrefillWorkload("chunk", B, n_new, H, d_h, r, dtype, int(rng.integers(1 << 30))))
    out = {k: _store(v, dtype) for k, v in cache.items()}
    out.update(new)
    out["starts"] = starts
    out["capacity"] = T
    return out



def projection_inputs(*, batch: int, n_new: int, d_model: int, heads: int, head_dim: int, rank: int,
                      dtype: str, seed: int) -> dict:
    """Inputs of the fused projection + append: hidden states X [B, n, d] ~ N(0, 1)
    and the key/value projection weights W^K_shared, W^V_shared [d, d_h] and
    U^K, U^V [H, d, r] ~ N(0, 1/d), so every projected feature has unit
    variance, like the cache rows of the decode workloads."""
    rng = np.random.default_rng(seed)
    B, n, d, H, d_h, r = batch, n_new, d_model, heads, head_dim, rank
    w_std = np.float32(1.0 / np.sqrt(d))
    x = rng.standard_normal((B, n, d), dtype=np.float32)
    wk = rng.standard_normal((d, d_h), dtype=np.float32) * w_std
    wv = rng.standard_normal((d, d_h), dtype=np.float32) * w_std
    uk = rng.standard_normal((H, d, r), dtype=np.float32) * w_std
    uv = rng.standard_normal((H, d, r), dtype=np.float32) * w_std
    return dict(x=_store(x, dtype), wk=_store(wk, dtype), wv=_store(wv, dtype), uk=_store(uk, dtype),
                uv=_store(uv, dtype), dtype=dtype, heads=H, head_dim=d_h, rank=r, d_model=d)


def mha_inputs(*, batch: int, capacity: int, heads: int, head_dim: int, lens, dtype: str, seed: int) -> dict:
    """A plain per-head K/V cache for the MHA baseline: q [B, H, d_h], k and v
    [B, T, H, d_h], all N(0, 1) up to each sequence's length, zero beyond."""
    rng = np.random.default_rng(seed)
    B, T, H, d_h = batch, capacity, heads, head_dim
    seq_lens = np.asarray(lens, dtype=np.int32)
    assert seq_lens.shape == (B,) and int(seq_lens.max(initial=0)) <= T
    sdt = np.uint16 if dtype == "bf16" else np.float32
    q = _store(rng.standard_normal((B, H, d_h), dtype=np.float32), dtype)
    k = np.zeros((B, T, H, d_h), sdt)
    v = np.zeros((B, T, H, d_h), sdt)
    for b in range(B):
        n = int(seq_lens[b])
        k[b, :n] = _store(rng.standard_normal((n, H, d_h), dtype=np.float32), dtype)
        v[b, :n] = _store(rng.standard_normal((n, H, d_h), dtype=np.float32), dtype)
    return dict(q=q, k=k, v=v, seq_lens=seq_lens, dtype=dtype)
