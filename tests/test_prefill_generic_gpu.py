"""lrkv_prefill and lrkv_prefill_chunk outside the rank 0/8/16/32 MFMA
kernel's envelope, through the C ABI, against the float64 oracle: bf16 at
the other ranks up to 128 on the padded MFMA kernel (prefill_wide_kernel:
every even rank; odd ranks with an even number of heads whose windows fit),
fp32 and the rest on the vector-ALU kernel (prefill_generic_kernel).

Bar: max |gpu - oracle| <= 1e-5 * ||oracle||_inf for fp32 storage and
2e-2 * ||oracle||_inf for bf16 storage.  Element by element, at sizes that
span several 32-query blocks and key tiles with ragged tails.
"""
import numpy as np
import pytest
import torch

import oracle as O
import rank_compressed_kv_lrkv_amd as L
from rank_compressed_kv_lrkv_amd.workloads import PrefillWorkload, as_f64, chunk_inputs, prefill_inputs
from tests.gpu_util import TOL, TORCH_DT, err_ratio, say, to_dev

pytestmark = pytest.mark.gpu
NEW = ("k_s", "v_s", "z_k", "z_v")

SHAPES = [
    # name, dtype, batch, seq_len, heads, head_dim, rank
    ("f32_r16", "f32", 2, 100, 8, 128, 16),
    ("f32_r54_h32", "f32", 1, 70, 32, 128, 54),
    ("f32_r0_dh64", "f32", 1, 65, 4, 64, 0),
    ("f32_dh16_r5", "f32", 2, 33, 3, 16, 5),
    ("f32_L1", "f32", 1, 1, 4, 128, 16),
    ("bf16_r54_h32", "bf16", 2, 130, 32, 128, 54),
    ("bf16_r55_h18", "bf16", 1, 97, 18, 128, 55),
    ("bf16_r128_h6", "bf16", 1, 64, 6, 128, 128),
    ("bf16_r46_h12", "bf16", 1, 40, 12, 128, 46),
    ("bf16_r51_h12", "bf16", 2, 31, 12, 128, 51),
    ("bf16_dh32_r16", "bf16", 1, 50, 4, 32, 16),
    ("bf16_r64_dh64_h5", "bf16", 2, 77, 5, 64, 64),
    ("bf16_r34_h8", "bf16", 1, 130, 8, 128, 34),
    ("bf16_r54_L1", "bf16", 1, 1, 4, 128, 54),
    ("bf16_r66_h4", "bf16", 1, 70, 4, 128, 66),
    ("bf16_r96_dh64_h7", "bf16", 2, 45, 7, 64, 96),
    ("bf16_r127_h3", "bf16", 1, 40, 3, 128, 127),
    ("bf16_r55_h9", "bf16", 1, 60, 9, 128, 55),
    ("bf16_r126_h4", "bf16", 1, 33, 4, 128, 126),
    ("bf16_r121_h2", "bf16", 1, 40, 2, 128, 121),
    ("bf16_r123_h2", "bf16", 1, 40, 2, 128, 123),
    ("bf16_r5_dh64_h4", "bf16", 2, 50, 4, 64, 5),
    ("bf16_r51_h6_dh64", "bf16", 1, 90, 6, 64, 51),
]


def expected_kernel(dt, d_h, r, H):
    """bf16 at head_dim 64/128 and a rank other than 0/8/16/32 runs on the
    padded MFMA kernel: an even rank always, an odd one with an even number
    of heads when every head's window (r plus (w r) mod 8, w < 4) fits in
    128 rows; the rest on the vector ALUs."""
    if dt == "bf16" and d_h in (64, 128) and 1 <= r <= 128:
        if r % 2 == 0:
            return "prefill_wide_kernel"
        if H % 2 == 0 and max(r + ((w * r) & 7) for w in range(4)) <= 128:
            return "prefill_wide_kernel"
    return "prefill_generic_kernel"


def f64(d, k):
    return as_f64(d[k], d["dtype"])


@pytest.mark.parametrize("name,dt,B,Lq,H,d_h,r", SHAPES, ids=[s[0] for s in SHAPES])
def test_prefill_generic(name, dt, B, Lq, H, d_h, r):
    kern = expected_kernel(dt, d_h, r, H)
    assert L.lrkv_prefill_kernel(TORCH_DT[dt], H, d_h, r) == kern
    say(f"case prefill ({kern}) {name}")
    d = prefill_inputs(PrefillWorkload(name, B, Lq, H, d_h, r, dt, 1000 + H + r))
    t = {k: to_dev(d[k], dt) for k in ("q",) + NEW + ("b_k", "b_v")}
    out = L.lrkv_prefill(t["q"], t["k_s"], t["v_s"], t["z_k"], t["z_v"], t["b_k"], t["b_v"])
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    want = O.prefill(f64(d, "q"), f64(d, "k_s"), f64(d, "v_s"), f64(d, "z_k"), f64(d, "z_v"), f64(d, "b_k"),
                     f64(d, "b_v"))
    e = err_ratio(got, want)
    say(f"  {name}: err/||out||inf = {e:.3e} (tol {TOL[dt]:.0e})")
    assert np.all(np.isfinite(got)) and e <= TOL[dt], (name, e)


def test_prefill_generic_writes_cache():
    """With cache pointers the tokens land bit-exactly in slots [0, L), the
    slots after them untouched."""
    dt, B, Lq, H, d_h, r, cap = "f32", 2, 45, 6, 64, 54, 64
    say("case prefill (vector ALU) with the cache written, fp32 r54")
    d = prefill_inputs(PrefillWorkload("cache", B, Lq, H, d_h, r, dt, 77))
    t = {k: to_dev(d[k], dt) for k in ("q",) + NEW + ("b_k", "b_v")}
    sentinel = 12345.0
    cache = L.LrkvCache(*(torch.full((B, cap) + tuple(t[k].shape[2:]), sentinel, dtype=torch.float32, device="cuda")
                          for k in NEW))
    L.lrkv_prefill(t["q"], t["k_s"], t["v_s"], t["z_k"], t["z_v"], t["b_k"], t["b_v"], cache=cache)
    torch.cuda.synchronize()
    for k, c in zip(NEW, (cache.k_s, cache.v_s, cache.z_k, cache.z_v)):
        assert torch.equal(c[:, :Lq], t[k]), k
        assert bool((c[:, Lq:] == sentinel).all()), k


CHUNKS = [
    # name, dtype, batch, heads, head_dim, rank, capacity, starts, n_new
    ("f32_r16", "f32", 3, 8, 128, 16, 320, [0, 37, 190], 100),
    ("bf16_r54", "bf16", 2, 32, 128, 54, 200, [64, 5], 33),
    ("bf16_r46_long", "bf16", 2, 12, 128, 46, 700, [600, 130], 64),
    ("bf16_r128", "bf16", 2, 6, 128, 128, 160, [100, 7], 40),
    ("bf16_r51_h12", "bf16", 2, 12, 128, 51, 300, [250, 3], 37),
    ("bf16_r55_h9", "bf16", 1, 9, 128, 55, 120, [70], 20),
    ("bf16_r55_one_token", "bf16", 2, 18, 128, 55, 300, [299, 0], 1),
]


@pytest.mark.parametrize("name,dt,B,H,d_h,r,cap,starts,n", CHUNKS, ids=[c[0] for c in CHUNKS])
def test_prefill_chunk_generic(name, dt, B, H, d_h, r, cap, starts, n):
    say(f"case prefill chunk ({expected_kernel(dt, d_h, r, H)}) {name} starts={starts} n_new={n}")
    d = chunk_inputs(batch=B, heads=H, head_dim=d_h, rank=r, capacity=cap, starts=starts, n_new=n, seed=40 + r,
                     dtype=dt)
    cache = L.LrkvCache(*(to_dev(d["cache_" + k], dt) for k in NEW))
    start = torch.from_numpy(np.asarray(starts, np.int32)).cuda()
    t = {k: to_dev(d[k], dt) for k in ("q",) + NEW + ("b_k", "b_v")}
    out = L.lrkv_prefill_chunk(cache, start, max(starts), t["q"], t["k_s"], t["v_s"], t["z_k"], t["z_v"], t["b_k"],
                               t["b_v"])
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    c = {k: as_f64(d["cache_" + k], dt).copy() for k in NEW}
    for b, s0 in enumerate(starts):
        for k in NEW:
            c[k][b, s0:s0 + n] = f64(d, k)[b]
    want = O.prefill_with_past(f64(d, "q"), c["k_s"], c["v_s"], c["z_k"], c["z_v"], f64(d, "b_k"), f64(d, "b_v"),
                               d["starts"])
    e = err_ratio(got, want)
    say(f"  {name}: err/||out||inf = {e:.3e} (tol {TOL[dt]:.0e})")
    assert np.all(np.isfinite(got)) and e <= TOL[dt], (name, e)


@pytest.mark.parametrize("wname", ["prefill_bf16_L4k_r54", "prefill_bf16_L4k_r128", "prefill_bf16_L4k_r55",
                                   "prefill_bf16_L4k_h9_r55"])
def test_prefill_trained_ranks_full_size_sampled_rows(wname):
    """The 4096-token workloads at trained ranks, at full size (the windowed
    MFMA kernel at ranks 54, 55 and 128; the vector-ALU kernel at rank 55
    with 9 heads):
    sampled query rows, each computed by the oracle as a decode over its
    causal prefix."""
    from rank_compressed_kv_lrkv_amd.workloads import PREFILL_WORKLOADS
    wl = PREFILL_WORKLOADS[wname]
    say(f"case {wl} (full size, sampled rows, {L.lrkv_prefill_kernel(torch.bfloat16, wl.heads, wl.head_dim, wl.rank)})")
    d = prefill_inputs(wl)
    t = {k: to_dev(d[k], "bf16") for k in ("q",) + NEW + ("b_k", "b_v")}
    out = L.lrkv_prefill(t["q"], t["k_s"], t["v_s"], t["z_k"], t["z_v"], t["b_k"], t["b_v"])
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got))
    b_k, b_v = f64(d, "b_k"), f64(d, "b_v")
    H = wl.heads
    for h in (0, H // 2, H - 1):
        for i in (0, 1, 31, 32, 33, 1000, 2047, 4095):
            n = i + 1
            want = O.decode(f64(d, "q")[0:1, i][:, [h]], f64(d, "k_s")[0:1, :n], f64(d, "v_s")[0:1, :n],
                            f64(d, "z_k")[0:1, :n][:, :, [h]], f64(d, "z_v")[0:1, :n][:, :, [h]], b_k[[h]], b_v[[h]],
                            [n])[0, 0]
            e = float(np.max(np.abs(got[0, i, h] - want)) / np.max(np.abs(want)))
            say(f"  h={h} row={i}: err/||row||inf = {e:.3e}")
            assert e <= TOL["bf16"], (h, i, e)
