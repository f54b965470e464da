"""Decode at the ranks the LRKV slides sweep ("The rank directly sets the
theoretical cache budget", Table 7; "Backup: the complete rank sweep
clarifies the trade-off", Table 8), where a token's latent run of H*r
elements is not a whole number of 16-byte chunks: the any-rank scans
(decode_mfma_any_kernel, the bf16 default at head_dim 128, and
decode_generic_kernel) through the C ABI against the float64 oracle, and
the cache append at those ranks, bit-exact.

Bar: max |gpu - oracle| <= 1e-5 * ||oracle||_inf (fp32 storage) or
2e-2 * ||oracle||_inf (bf16 storage), as every decode test.
"""
import numpy as np
import pytest
import torch

import rank_compressed_kv_lrkv_amd as L
from rank_compressed_kv_lrkv_amd.workloads import DECODE_WORKLOADS, DecodeWorkload, decode_inputs
from tests.gpu_util import TOL, TORCH_DT, device_cache, err_ratio, from_dev, oracle_decode, run_decode, say, to_dev

pytestmark = pytest.mark.gpu

PAGE_SHAPES = [(32, 54, 128), (18, 55, 128), (6, 128, 128)]   # (heads, rank, head_dim)


def check(d, got, name, batches=None, heads=None):
    want = oracle_decode(d, batches, heads)
    sub = got
    if batches is not None or heads is not None:
        sub = got[np.ix_(list(batches if batches is not None else range(got.shape[0])),
                         list(heads if heads is not None else range(got.shape[1])))]
    e = err_ratio(sub, want)
    say(f"  {name}: err/||out||inf = {e:.3e} (tol {TOL[d['dtype']]:.0e})")
    assert np.all(np.isfinite(sub)) and e <= TOL[d["dtype"]], (name, e)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("H,r,d_h", PAGE_SHAPES, ids=[f"H{h}_r{r}_dh{d}" for h, r, d in PAGE_SHAPES])
def test_page_ranks_full(H, r, d_h, dt):
    name = f"H{H}_r{r}_dh{d_h}_{dt}"
    want = "decode_mfma_any_kernel" if dt == "bf16" else "decode_generic_kernel"
    assert L.lrkv_decode_scan_kernel(TORCH_DT[dt], H, d_h, r) == want
    lens = np.array([700, 333, 1, 65], np.int32)           # several tiles, a ragged tail, one token
    say(f"case {name} lens={lens.tolist()} ({want})")
    d = decode_inputs(DecodeWorkload(name, 4, H, d_h, r, 700, dt, 4711 + H + r), lens=lens)
    check(d, run_decode(d), name)
    check(d, run_decode(d, split_tokens=128), name + " split 128")
    if dt == "bf16":
        other = 3 if want == "decode_mfma_any_kernel" else 4
        say(f"case {name} on engine {other}")
        check(d, run_decode(d, engine=other), f"{name} engine {other}")
        check(d, run_decode(d, engine=other, split_tokens=128), f"{name} engine {other} split 128")


# (heads, rank) for the any-rank MFMA scan: every window size (4 to 32 words
# per lane), odd ranks (windows starting mid-word for odd heads), 1, 2, 4 and
# 8 heads (four column copies per head), 9-16 heads (two), 17-31 heads (one,
# idle lanes), more than 32 (a partial second group of heads), an odd head
# count at an even rank, and the ranks the tuned scans also take.
MFMA_ANY_SHAPES = [(2, 9), (4, 12), (6, 13), (32, 17), (8, 23), (32, 31), (10, 33), (12, 46), (12, 51),
                   (32, 54), (18, 55), (16, 63), (4, 65), (40, 51), (33, 54), (2, 77), (6, 96), (2, 101),
                   (2, 127), (6, 128), (32, 16), (64, 32), (16, 128), (8, 54), (20, 128), (1, 40)]


@pytest.mark.parametrize("H,r", MFMA_ANY_SHAPES, ids=[f"H{h}_r{r}" for h, r in MFMA_ANY_SHAPES])
def test_mfma_any_rank_sweep(H, r):
    """The any-rank MFMA scan (engine 4) at bf16, head_dim 128: several tiles
    per wave, ragged tails, one token, an empty sequence; default split and
    two fixed ones."""
    name = f"H{H}_r{r}_mfma_any"
    lens = np.array([300, 97, 1, 0, 33], np.int32)
    say(f"case {name} lens={lens.tolist()}")
    d = decode_inputs(DecodeWorkload(name, 5, H, 128, r, 300, "bf16", 900 + 7 * H + r), lens=lens)
    live = [0, 1, 2, 4]
    for split in (0, 128, 256):
        got = run_decode(d, engine=4, split_tokens=split)
        assert np.all(got[3] == 0), "empty sequence"
        check(d, got, f"{name} split {split}", batches=live)


@pytest.mark.parametrize("B,H,r", [(19, 32, 54), (3, 1024, 8), (9, 96, 21), (17, 128, 10)],
                         ids=["B19_H32_r54", "B3_H1024_r8", "B9_H96_r21", "B17_H128_r10"])
def test_mfma_any_batches_and_many_heads(B, H, r):
    """The any-rank MFMA scan with more than eight sequences (several
    workgroup rows of the absorbed-query kernel, one of them partial) and with
    many head groups, up to the 1024-head limit; ragged lengths."""
    rng = np.random.default_rng(7 * B + H + r)
    lens = rng.integers(1, 260, size=B).astype(np.int32)
    lens[B // 2] = 0
    name = f"B{B}_H{H}_r{r}_mfma_any"
    say(f"case {name} lens={lens.tolist()}")
    d = decode_inputs(DecodeWorkload(name, B, H, 128, r, 260, "bf16", 77 * B + H + r), lens=lens)
    live = [b for b in range(B) if lens[b] > 0]
    for split in (0, 128):
        got = run_decode(d, engine=4, split_tokens=split)
        assert np.all(got[B // 2] == 0), "empty sequence"
        check(d, got, f"{name} split {split}", batches=live)


@pytest.mark.parametrize("H,r", [(7, 55), (20, 128)], ids=["H7_r55", "H20_r128"])
def test_any_rank_default_vector_scan_shapes(H, r):
    """bf16 shapes the default leaves on the any-rank vector scan: an odd
    heads * rank (token runs not on 4-byte boundaries), and 32-word windows
    with fewer than 32 heads."""
    assert L.lrkv_decode_scan_kernel(torch.bfloat16, H, 128, r) == "decode_generic_kernel"
    lens = np.array([300, 97, 1], np.int32)
    say(f"case H{H}_r{r} default engine lens={lens.tolist()}")
    d = decode_inputs(DecodeWorkload(f"H{H}_r{r}", 3, H, 128, r, 300, "bf16", 31 * H + r), lens=lens)
    check(d, run_decode(d), f"H{H} r{r} default")
    if H * r % 2 == 0:
        check(d, run_decode(d, engine=4), f"H{H} r{r} engine 4")


def test_mfma_any_phases_and_tail_tiles():
    """Scan and merge called apart (lrkv_decode_partial / lrkv_decode_combine
    through engine 4), at lengths that leave every wave of a split a
    different number of tiles and a partial last tile."""
    H, r = 12, 51
    lens = np.array([1, 31, 32, 33, 127, 128, 129, 511], np.int32)
    d = decode_inputs(DecodeWorkload("phases", len(lens), H, 128, r, 512, "bf16", 4242), lens=lens)
    cache = device_cache(d)
    dl = torch.from_numpy(lens).cuda()
    q, bk, bv = (to_dev(d[k], "bf16") for k in ("q", "b_k", "b_v"))
    for split in (0, 128, 512):
        call = L.DecodeCall(cache, dl, 512, q, bk, bv, split_tokens=split, engine=4)
        call.partial()
        call.combine()
        torch.cuda.synchronize()
        say(f"case phases H{H} r{r} split {split}")
        check(d, from_dev(call.out), f"phases split {split}")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_page_rank_long_context_sampled(dt):
    """The 8K-context shape of the bandwidth workload (d_h = 128, 32 heads) at
    the pages' rank 54, with the library's default split, sampled pairs."""
    H, r, d_h, T = 32, 54, 128, 8192
    say(f"case H{H}_r{r}_dh{d_h}_T{T}_{dt} batch=3 (sampled)")
    d = decode_inputs(DecodeWorkload("rank54_T8k", 3, H, d_h, r, T, dt, 99), lens=np.array([8192, 5000, 8191], np.int32))
    got = run_decode(d)
    for b, h in ((0, 0), (1, 17), (2, 31)):
        check(d, got, f"b={b} h={h}", [b], [h])


@pytest.mark.parametrize("name", ["tiny_f32_T64", "small_bf16_T2k"])
def test_any_rank_engine_on_tuned_shapes(name):
    """The any-rank scan (engine 3) on shapes the tuned scans take."""
    wl = DECODE_WORKLOADS[name]
    lens = None if name == "tiny_f32_T64" else np.array([2048, 1000, 1, 64, 65, 2047, 7, 1500], np.int32)
    say(f"case {name} on the any-rank scan")
    d = decode_inputs(wl, lens=lens)
    check(d, run_decode(d, engine=3), name + " engine 3")


def test_any_rank_many_heads():
    """More than 32 heads: the grid runs a second group of heads."""
    H, r, d_h = 40, 20, 64
    d = decode_inputs(DecodeWorkload("many_heads", 2, H, d_h, r, 300, "bf16", 5), lens=np.array([300, 97], np.int32))
    say("case H40_r20_dh64_bf16")
    check(d, run_decode(d), "H40 r20")


def test_rank_zero_and_empty_sequence_any_rank():
    H, r, d_h = 6, 0, 64
    d = decode_inputs(DecodeWorkload("mqa", 3, H, d_h, r, 130, "f32", 6), lens=np.array([130, 0, 1], np.int32))
    got = run_decode(d, engine=3)
    say("case rank 0 on the any-rank scan, an empty sequence")
    assert np.all(got[1] == 0)
    check(d, got, "rank 0", batches=[0, 2])


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_append_then_decode_odd_latent_run(dt):
    """Append at H*r = 990 elements per token (not whole 16-byte chunks):
    bit-exact slots, untouched neighbours, then decode of the appended cache."""
    B, H, r, d_h, T = 2, 18, 55, 128, 200
    lens = np.array([200, 130], np.int32)
    d = decode_inputs(DecodeWorkload("append55", B, H, d_h, r, T, dt, 77), lens=lens)
    tdt = TORCH_DT[dt]
    cache = L.LrkvCache.empty(B, H, d_h, r, T, dtype=tdt)
    for t in (cache.k_s, cache.v_s, cache.z_k, cache.z_v):
        t.fill_(-5.0)
    filled = np.zeros(B, np.int32)
    for n in (64, 1, 37, 100, 64):
        rows = {k: np.zeros((B, n) + d[k].shape[2:], d[k].dtype) for k in ("k_s", "v_s", "z_k", "z_v")}
        for b in range(B):
            m = int(min(n, T - filled[b]))
            for k in rows:
                rows[k][b, :m] = d[k][b, filled[b]:filled[b] + m]
        L.lrkv_append(cache, torch.from_numpy(filled.copy()).cuda(), *(to_dev(rows[k], dt) for k in rows))
        filled = np.minimum(filled + n, T)
    torch.cuda.synchronize()
    view = np.int16 if dt == "bf16" else np.int32
    for k, t in (("k_s", cache.k_s), ("v_s", cache.v_s), ("z_k", cache.z_k), ("z_v", cache.z_v)):
        got = t.view(torch.int16 if dt == "bf16" else torch.int32).cpu().numpy()
        assert np.array_equal(got, np.ascontiguousarray(d[k]).view(view)), k
    say(f"case append H18 r55 {dt}: bit-exact")
    check(d, run_decode(d, cache=cache), f"decode after append {dt}")
