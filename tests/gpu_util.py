"""Helpers for the GPU parity tests: move seeded workload arrays to the
device, run the library, and compare with the float64 oracle."""
import sys

import numpy as np
import torch

import oracle as O
import rank_compressed_kv_lrkv_amd as L
from rank_compressed_kv_lrkv_amd.workloads import as_f64

TOL = {"f32": 1e-5, "bf16": 2e-2}
TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(arr, dtype):
    """Stored workload array (float32 values or bf16 bit patterns) -> device tensor."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.cuda()


def from_dev(t):
    return t.float().cpu().numpy().astype(np.float64)


def device_cache(d):
    dt = d["dtype"]
    return L.LrkvCache(to_dev(d["k_s"], dt), to_dev(d["v_s"], dt), to_dev(d["z_k"], dt), to_dev(d["z_v"], dt))


def run_decode(d, split_tokens=0, max_len=None, cache=None, engine=0):
    dt = d["dtype"]
    cache = cache if cache is not None else device_cache(d)
    lens = torch.from_numpy(np.asarray(d["seq_lens"], np.int32)).cuda()
    ml = int(d["capacity"] if max_len is None else max_len)
    out = L.lrkv_decode(cache, lens, ml, to_dev(d["q"], dt), to_dev(d["b_k"], dt), to_dev(d["b_v"], dt),
                        split_tokens=split_tokens, engine=engine)
    torch.cuda.synchronize()
    return from_dev(out)


def oracle_decode(d, batches=None, heads=None):
    """float64 oracle on a subset of (sequence, head) pairs; returns [len(batches), len(heads), d_h]."""
    dt = d["dtype"]
    B, H = d["q"].shape[0], d["q"].shape[1]
    bs = list(range(B)) if batches is None else list(batches)
    hs = list(range(H)) if heads is None else list(heads)
    f = lambda k: as_f64(d[k], dt)
    lens = np.asarray(d["seq_lens"])[bs]
    T = int(max(lens.max(initial=0), 1))
    q = f("q")[bs][:, hs]
    k_s = as_f64(d["k_s"][bs, :T], dt)
    v_s = as_f64(d["v_s"][bs, :T], dt)
    z_k = as_f64(d["z_k"][bs, :T][:, :, hs], dt)
    z_v = as_f64(d["z_v"][bs, :T][:, :, hs], dt)
    return O.decode(q, k_s, v_s, z_k, z_v, f("b_k")[hs], f("b_v")[hs], lens)


def err_ratio(got, want):
    """max |got - want| / ||want||_inf."""
    return float(np.max(np.abs(got - want)) / max(np.max(np.abs(want)), 1e-30))


def check_decode_after_append(seed=21):
    """Fill an empty cache by several appends at per-sequence positions, then
    decode; the logical cache is what the oracle sees."""
    from rank_compressed_kv_lrkv_amd.workloads import DecodeWorkload, decode_inputs
    B, H, d_h, r, T, dt = 3, 8, 64, 16, 300, "bf16"
    lens = np.array([300, 171, 65], np.int32)
    d = decode_inputs(DecodeWorkload("appended", B, H, d_h, r, T, dt, seed), lens=lens)
    cache = L.LrkvCache.empty(B, H, d_h, r, T, dtype=torch.bfloat16)
    filled = np.zeros(B, np.int32)
    step = 0
    while np.any(filled < lens):
        n = [64, 1, 37, 100][step % 4]
        step += 1
        rows = {k: np.zeros((B, n) + d[k].shape[2:], d[k].dtype) for k in ("k_s", "v_s", "z_k", "z_v")}
        for b in range(B):
            m = int(min(n, lens[b] - filled[b]))
            for k in rows:
                rows[k][b, :m] = d[k][b, filled[b]:filled[b] + m]
        pos = torch.from_numpy(filled.copy()).cuda()
        L.lrkv_append(cache, pos, *(to_dev(rows[k], dt) for k in ("k_s", "v_s", "z_k", "z_v")))
        filled = np.minimum(filled + n, lens)
        # rows appended past a sequence's length are zeros and lie beyond its length
    got = run_decode(d, cache=cache)
    want = oracle_decode(d)
    e = err_ratio(got, want)
    say(f"  decode after {step} appends: err/||out||inf = {e:.3e}")
    assert e <= TOL[dt]
