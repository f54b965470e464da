"""lrkv_prefill (bf16 MFMA, through the C ABI) against the float64 oracle.

Bar: max |gpu - oracle| <= 2e-2 * ||oracle||_inf (bf16 storage, fp32
accumulation).  Small shapes are compared element by element; the full
4096-token workload is compared on sampled query rows, each of which the
oracle computes as a decode over its causal prefix.
"""
import numpy as np
import pytest
import torch

import oracle as O
import rank_compressed_kv_lrkv_amd as L
from rank_compressed_kv_lrkv_amd.workloads import PREFILL_WORKLOADS, PrefillWorkload, as_f64, prefill_inputs
from tests.gpu_util import err_ratio, say, to_dev

pytestmark = pytest.mark.gpu
TOL = 2e-2


def run_prefill(d, cache=None):
    dt = d["dtype"]
    t = {k: to_dev(d[k], dt) for k in ("q", "k_s", "v_s", "z_k", "z_v", "b_k", "b_v")}
    out = L.lrkv_prefill(t["q"], t["k_s"], t["v_s"], t["z_k"], t["z_v"], t["b_k"], t["b_v"], cache=cache)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


def f64(d, k):
    return as_f64(d[k], d["dtype"])


def check_full(d, name):
    got = run_prefill(d)
    want = O.prefill(f64(d, "q"), f64(d, "k_s"), f64(d, "v_s"), f64(d, "z_k"), f64(d, "z_v"), f64(d, "b_k"),
                     f64(d, "b_v"))
    e = err_ratio(got, want)
    say(f"  {name}: err/||out||inf = {e:.3e}")
    assert np.all(np.isfinite(got)) and e <= TOL, (name, e)


SHAPES = [
    # name, batch, seq_len, heads, head_dim, rank
    ("L100_H8_r16", 2, 100, 8, 128, 16),
    ("L1", 1, 1, 4, 128, 16),
    ("L31_H6", 1, 31, 6, 128, 16),
    ("L33_H5_r8", 2, 33, 5, 128, 8),
    ("L96_r32", 1, 96, 4, 128, 32),
    ("L70_r0_mqa", 1, 70, 8, 128, 0),
    ("dh64_r16", 2, 65, 4, 64, 16),
    ("dh64_r32", 1, 64, 8, 64, 32),
]


@pytest.mark.parametrize("name,B,Lq,H,d_h,r", SHAPES, ids=[s[0] for s in SHAPES])
def test_prefill_small(name, B, Lq, H, d_h, r):
    say(f"case prefill {name}")
    d = prefill_inputs(PrefillWorkload(name, B, Lq, H, d_h, r, "bf16", 4242))
    check_full(d, name)


def test_prefill_workload_reduced():
    wl = PREFILL_WORKLOADS["prefill_bf16_L4k"]
    say(f"case {wl.name} batch=1 seq_len=512")
    d = prefill_inputs(wl, batch=1, seq_len=512, seed=8)
    check_full(d, "prefill 512")


def test_prefill_full_size_sampled_rows():
    wl = PREFILL_WORKLOADS["prefill_bf16_L4k"]
    say(f"case {wl} (full size, sampled rows)")
    d = prefill_inputs(wl)
    got = run_prefill(d)
    assert np.all(np.isfinite(got))
    b_k, b_v = f64(d, "b_k"), f64(d, "b_v")
    for b, h in ((0, 0), (3, 31), (2, 17)):
        hs = [h]
        rows = [0, 1, 31, 32, 33, 1000, 2047, 4095]
        for i in rows:
            n = i + 1
            want = O.decode(f64(d, "q")[b:b + 1, i][:, hs], as_f64(d["k_s"][b:b + 1, :n], "bf16"),
                            as_f64(d["v_s"][b:b + 1, :n], "bf16"), as_f64(d["z_k"][b:b + 1, :n][:, :, hs], "bf16"),
                            as_f64(d["z_v"][b:b + 1, :n][:, :, hs], "bf16"), b_k[hs], b_v[hs], [n])[0, 0]
            e = float(np.max(np.abs(got[b, i, h] - want)) / np.max(np.abs(want)))
            say(f"  b={b} h={h} row={i}: err/||row||inf = {e:.3e}")
            assert e <= TOL, (b, h, i, e)


def test_prefill_writes_cache_bit_exact():
    say("case prefill cache write")
    B, Lq, H, d_h, r, cap = 2, 77, 8, 128, 16, 96
    d = prefill_inputs(PrefillWorkload("cache", B, Lq, H, d_h, r, "bf16", 7))
    cache = L.LrkvCache.empty(B, H, d_h, r, cap, dtype=torch.bfloat16)
    fill = torch.full((), -3.0, dtype=torch.bfloat16)
    for t in (cache.k_s, cache.v_s, cache.z_k, cache.z_v):
        t.fill_(fill.item())
    run_prefill(d, cache=cache)
    for k, t in (("k_s", cache.k_s), ("v_s", cache.v_s), ("z_k", cache.z_k), ("z_v", cache.z_v)):
        got = t.view(torch.int16).cpu().numpy()
        assert np.array_equal(got[:, :Lq], np.ascontiguousarray(d[k]).view(np.int16)), k
        assert np.all(got[:, Lq:] == np.int16(fill.view(torch.int16).item())), k
