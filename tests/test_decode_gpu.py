"""lrkv_decode (HIP, through the C ABI) against the float64 oracle.

Bar: max |gpu - oracle| <= tau * ||oracle||_inf with tau = 1e-5 (fp32 storage)
or 2e-2 (bf16 storage, fp32 accumulation), over the whole output tensor of
each case.  Full-size workloads are checked on sampled (sequence, head)
pairs that the oracle computes one by one; reduced sizes of the same
distributions are checked element by element.
"""
import numpy as np
import pytest
import torch

from rank_compressed_kv_lrkv_amd.workloads import DECODE_WORKLOADS, DecodeWorkload, decode_inputs
from tests.gpu_util import TOL, err_ratio, oracle_decode, run_decode, say

pytestmark = pytest.mark.gpu


def check(d, got, batches=None, heads=None, name=""):
    want = oracle_decode(d, batches, heads)
    sub = got if batches is None and heads is None else got[np.ix_(
        list(batches if batches is not None else range(got.shape[0])),
        list(heads if heads is not None else range(got.shape[1])))]
    e = err_ratio(sub, want)
    say(f"  {name}: err/||out||inf = {e:.3e} (tol {TOL[d['dtype']]:.0e})")
    assert e <= TOL[d["dtype"]], (name, e)
    return e


def test_tiny_f32_full():
    wl = DECODE_WORKLOADS["tiny_f32_T64"]
    say(f"case {wl}")
    d = decode_inputs(wl)
    check(d, run_decode(d), name=wl.name)


def test_small_bf16_full():
    wl = DECODE_WORKLOADS["small_bf16_T2k"]
    say(f"case {wl}")
    d = decode_inputs(wl)
    check(d, run_decode(d), name=wl.name)


def test_mid_bf16_reduced_ragged_tail():
    wl = DECODE_WORKLOADS["mid_bf16_T8k"]
    lens = np.array([1000, 999, 513, 1, 64, 65], np.int32)
    say(f"case {wl.name} batch=6 capacity=1000 lens={lens.tolist()}")
    d = decode_inputs(wl, batch=6, capacity=1000, lens=lens, seed=7)
    check(d, run_decode(d), name="mid reduced")


def test_mid_bf16_full_size_sampled():
    wl = DECODE_WORKLOADS["mid_bf16_T8k"]
    say(f"case {wl} (full size, sampled)")
    d = decode_inputs(wl)
    got = run_decode(d)
    assert np.all(np.isfinite(got))
    for b, h in ((0, 0), (7, 31), (18, 5), (31, 16), (31, 31)):
        check(d, got, [b], [h], name=f"mid full b={b} h={h}")


def test_ragged_reduced():
    wl = DECODE_WORKLOADS["ragged_bf16_T1k_64k"]
    lens = np.array([4096, 1, 63, 64, 65, 2047, 3000, 129], np.int32)
    say(f"case {wl.name} batch=8 capacity=4096 lens={lens.tolist()}")
    d = decode_inputs(wl, batch=8, capacity=4096, lens=lens, seed=11)
    check(d, run_decode(d), name="ragged reduced")


def test_ragged_full_size_sampled():
    wl = DECODE_WORKLOADS["ragged_bf16_T1k_64k"]
    say(f"case {wl} (full size, sampled)")
    d = decode_inputs(wl)
    got = run_decode(d)
    assert np.all(np.isfinite(got))
    lens = d["seq_lens"]
    bmax, bmin = int(np.argmax(lens)), int(np.argmin(lens))
    for b, h in ((bmax, 0), (bmax, 31), (bmin, 7), (5, 20)):
        check(d, got, [b], [h], name=f"ragged full b={b} len={lens[b]} h={h}")


@pytest.mark.parametrize("split", [64, 128, 960, 0, 4096])
def test_split_invariance(split):
    wl = DECODE_WORKLOADS["mid_bf16_T8k"]
    lens = np.array([4096, 3001, 700, 64], np.int32)
    say(f"case split={split} lens={lens.tolist()}")
    d = decode_inputs(wl, batch=4, capacity=4096, lens=lens, seed=3)
    check(d, run_decode(d, split_tokens=split), name=f"split {split}")


@pytest.mark.parametrize("batch,seed", [(70, 31), (130, 32)])
def test_balanced_partition_many_sequences(batch, seed):
    """The default partition of the MFMA scan is computed on the device from
    the lengths (more than one 64-sequence chunk here, with empty, one-token
    and tile-straddling sequences); the merge must find every sequence's
    items."""
    wl = DecodeWorkload("balanced", batch, 32, 64, 8, 300, "bf16", seed)
    rng = np.random.default_rng(seed)
    lens = rng.integers(0, 301, size=batch).astype(np.int32)
    lens[:4] = [0, 1, 300, 129]
    say(f"case balanced partition batch={batch} lens[:8]={lens[:8].tolist()} total={int(lens.sum())}")
    d = decode_inputs(wl, lens=lens, capacity=300)
    check(d, run_decode(d), name=f"balanced B={batch}")


@pytest.mark.parametrize("name", ["small_bf16_T2k", "mid_bf16_T8k"])
def test_deterministic_bitwise(name):
    wl = DECODE_WORKLOADS[name]
    say(f"case determinism {name}")
    d = decode_inputs(wl, seed=5, batch=4, capacity=2048, lens=np.array([2048, 1500, 3, 700], np.int32))
    a = run_decode(d)
    b = run_decode(d)
    assert np.array_equal(a, b)


EDGE = [
    # name, heads, head_dim, rank, dtype, lens
    ("single_token", 8, 64, 8, "bf16", [1, 1]),
    ("empty_and_short", 8, 64, 8, "bf16", [0, 3]),
    ("mqa_rank0", 8, 64, 0, "bf16", [300, 77]),
    ("one_head", 1, 128, 16, "bf16", [500, 64]),
    ("heads_64", 64, 64, 8, "bf16", [200, 129]),
    ("heads_6", 6, 128, 16, "bf16", [333, 1]),
    ("heads_12_r32", 12, 128, 32, "bf16", [257, 190]),
    ("dh16_bf16", 4, 16, 8, "bf16", [100, 31]),
    ("dh32_r64", 8, 32, 64, "bf16", [90, 45]),
    ("f32_dh64", 8, 64, 8, "f32", [400, 1]),
    ("f32_dh128_r16", 4, 128, 16, "f32", [150, 66]),
    ("f32_rank4_g4", 16, 32, 4, "f32", [130, 64]),
    ("f32_rank0", 4, 16, 0, "f32", [64, 2]),
    # shapes of the MFMA scan (bf16, 32 or 64 heads): every rank it takes,
    # both head widths, lengths that end inside a tile and inside a wave's
    # share, empty and one-token sequences
    ("mfma_r0", 32, 128, 0, "bf16", [300, 33]),
    ("mfma_dh128_r8", 32, 128, 8, "bf16", [1, 257]),
    ("mfma_dh64_r8", 32, 64, 8, "bf16", [129, 1]),
    ("mfma_dh64_r16", 32, 64, 16, "bf16", [31, 0, 64]),
    ("mfma_dh64_r32", 32, 64, 32, "bf16", [95, 16]),
    ("mfma_h64_r32", 64, 128, 32, "bf16", [97, 200]),
    ("mfma_h64_r16", 64, 128, 16, "bf16", [160, 2]),
]


@pytest.mark.parametrize("name,H,d_h,r,dt,lens", EDGE, ids=[e[0] for e in EDGE])
def test_edge_shapes(name, H, d_h, r, dt, lens):
    wl = DecodeWorkload(name, len(lens), H, d_h, r, max(lens), dt, 1234)
    say(f"case {wl} lens={lens}")
    d = decode_inputs(wl, lens=np.array(lens, np.int32), capacity=max(max(lens), 1))
    check(d, run_decode(d), name=name)


def test_lengths_clamped_to_max_len():
    wl = DECODE_WORKLOADS["small_bf16_T2k"]
    say("case max_len clamp")
    d = decode_inputs(wl, batch=2, capacity=512, lens=np.array([512, 300], np.int32), seed=9)
    got = run_decode(d, max_len=256)            # the kernel sees at most 256 tokens per sequence
    d2 = dict(d, seq_lens=np.array([256, 256], np.int32))
    check(d2, got, name="clamped")


@pytest.mark.parametrize("name,split", [("mid_bf16_T8k", 0), ("mid_bf16_T8k", 256), ("small_bf16_T2k", 0)])
def test_partial_then_combine_equals_decode(name, split):
    # lrkv_decode_partial followed by lrkv_decode_combine on the same workspace
    # is the same computation as lrkv_decode: bitwise the same output
    import rank_compressed_kv_lrkv_amd as L
    from tests.gpu_util import device_cache, to_dev
    wl = DECODE_WORKLOADS[name]
    say(f"case partial + combine {name} split={split}")
    d = decode_inputs(wl, seed=9, batch=5, capacity=1200, lens=np.array([1200, 1, 640, 0, 999], np.int32))
    dt = d["dtype"]
    cache = device_cache(d)
    lens = torch.from_numpy(np.asarray(d["seq_lens"], np.int32)).cuda()
    q, b_k, b_v = to_dev(d["q"], dt), to_dev(d["b_k"], dt), to_dev(d["b_v"], dt)
    ws = L.decode_workspace(cache, 1200, split)
    both = L.lrkv_decode(cache, lens, 1200, q, b_k, b_v, split_tokens=split, workspace=ws)
    out = torch.full_like(both, 7.0)
    L.lrkv_decode(cache, lens, 1200, q, b_k, b_v, split_tokens=split, out=out, workspace=ws, phase="partial")
    L.lrkv_decode(cache, lens, 1200, q, b_k, b_v, split_tokens=split, out=out, workspace=ws, phase="combine")
    torch.cuda.synchronize()
    a, b = both.float().cpu().numpy(), out.float().cpu().numpy()
    assert np.array_equal(a, b)
    check(d, a.astype(np.float64), name=f"{name} split={split}")


@pytest.mark.parametrize("batch,length", [(5, 700), (3, 1), (40, 130), (7, 2048)])
def test_balanced_partition_uniform_lengths(batch, length):
    # every length equal: the partition in closed form (the same items as the general search)
    wl = DECODE_WORKLOADS["mid_bf16_T8k"]
    say(f"case balanced uniform batch={batch} length={length}")
    d = decode_inputs(wl, seed=40 + batch, batch=batch, capacity=length,
                      lens=np.full(batch, length, np.int32))
    check(d, run_decode(d), name=f"uniform B={batch} L={length}")


def test_vector_alu_scan_on_headline_shape():
    # lrkv_decode_ex(engine=1) runs the vector-ALU scan on a shape whose
    # default is the MFMA scan; both are held to the oracle
    import torch
    import rank_compressed_kv_lrkv_amd as L
    from tests.gpu_util import device_cache, from_dev, to_dev
    wl = DECODE_WORKLOADS["mid_bf16_T8k"]
    lens = np.array([1000, 999, 513, 1, 64, 65], np.int32)
    say(f"case {wl.name} engine=1 batch=6 capacity=1000 lens={lens.tolist()}")
    d = decode_inputs(wl, batch=6, capacity=1000, lens=lens, seed=17)
    cache = device_cache(d)
    lt = torch.from_numpy(lens).cuda()
    args = (cache, lt, 1000, to_dev(d["q"], "bf16"), to_dev(d["b_k"], "bf16"), to_dev(d["b_v"], "bf16"))
    for engine in (1, 2):
        out = L.lrkv_decode(*args, engine=engine)
        torch.cuda.synchronize()
        check(d, from_dev(out), name=f"engine {engine}")


def test_vector_alu_scan_full_headline_sampled():
    import torch
    import rank_compressed_kv_lrkv_amd as L
    from tests.gpu_util import device_cache, from_dev, to_dev
    wl = DECODE_WORKLOADS["mid_bf16_T8k"]
    say(f"case {wl} engine=1 (full size, sampled)")
    d = decode_inputs(wl)
    cache = device_cache(d)
    lt = torch.from_numpy(np.asarray(d["seq_lens"], np.int32)).cuda()
    out = L.lrkv_decode(cache, lt, wl.capacity, to_dev(d["q"], "bf16"), to_dev(d["b_k"], "bf16"),
                        to_dev(d["b_v"], "bf16"), engine=1)
    torch.cuda.synchronize()
    got = from_dev(out)
    assert np.all(np.isfinite(got))
    for b, h in ((0, 0), (31, 31), (17, 9)):
        check(d, got, [b], [h], name=f"vector scan full b={b} h={h}")
