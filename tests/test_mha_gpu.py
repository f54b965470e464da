"""lrkv_mha_decode (HIP, through the C ABI), the plain multi-head baseline,
against the float64 oracle's textbook attention per (sequence, head)."""
import numpy as np
import pytest
import torch

import oracle as O
import rank_compressed_kv_lrkv_amd as L
from rank_compressed_kv_lrkv_amd.workloads import as_f64, mha_inputs
from tests.gpu_util import TOL, err_ratio, from_dev, say, to_dev

pytestmark = pytest.mark.gpu


def oracle_mha(d, scale=None):
    dt = d["dtype"]
    q, k, v = as_f64(d["q"], dt), as_f64(d["k"], dt), as_f64(d["v"], dt)
    B, H, d_h = q.shape
    sc = 1.0 / np.sqrt(d_h) if scale is None else scale
    out = np.zeros((B, H, d_h))
    for b in range(B):
        n = int(d["seq_lens"][b])
        for h in range(H):
            out[b, h] = O.softmax_attention(q[b, h], k[b, :n, h], v[b, :n, h], sc)
    return out


def run(d, max_len, split=0, scale=None):
    dt = d["dtype"]
    lens = torch.from_numpy(np.asarray(d["seq_lens"], np.int32)).cuda()
    out = L.lrkv_mha_decode(to_dev(d["k"], dt), to_dev(d["v"], dt), lens, max_len, to_dev(d["q"], dt), scale=scale,
                            split_tokens=split)
    torch.cuda.synchronize()
    return from_dev(out)


@pytest.mark.parametrize("dt,H,d_h,lens,split", [
    ("bf16", 32, 128, [1100, 777, 1, 64, 65], 0),
    ("bf16", 32, 128, [1100, 777, 1, 64, 65], 256),
    ("bf16", 8, 64, [300, 0, 129], 64),          # an empty sequence, a ragged tail
    ("bf16", 40, 128, [200, 513], 128),          # two head groups, the second partly filled
    ("f32", 5, 64, [97, 256, 31], 64),
    ("f32", 4, 128, [70, 3], 0),
])
def test_mha_decode_parity(dt, H, d_h, lens, split):
    say(f"case mha {dt} H={H} d_h={d_h} lens={lens} split={split}")
    T = max(lens) + 7
    d = mha_inputs(batch=len(lens), capacity=T, heads=H, head_dim=d_h, lens=lens, dtype=dt, seed=31 + H + d_h)
    got = run(d, max(lens), split)
    want = oracle_mha(d)
    assert err_ratio(got, want) <= TOL[dt]
    for b, n in enumerate(lens):
        if n == 0:
            assert np.all(got[b] == 0)


def test_mha_decode_scale_and_splits_agree():
    say("case mha scale, split invariance")
    d = mha_inputs(batch=2, capacity=600, heads=32, head_dim=128, lens=[600, 333], dtype="bf16", seed=5)
    want = oracle_mha(d, scale=0.05)
    for split in (64, 192, 0, 1024):
        assert err_ratio(run(d, 600, split, scale=0.05), want) <= TOL["bf16"], split


def test_mha_decode_headline_shape_sampled():
    # the matched-shape baseline of the benchmark: 32 sequences x 8192 tokens,
    # H = 32, d_h = 128 (4.3 GB of cache), seeded on the device; sampled
    # (sequence, head) pairs against the oracle
    say("case mha headline shape sampled")
    B, T, H, d_h = 32, 8192, 32, 128
    gen = torch.Generator(device="cuda").manual_seed(20261209)
    k = torch.randn(B, T, H, d_h, device="cuda", generator=gen).to(torch.bfloat16)
    v = torch.randn(B, T, H, d_h, device="cuda", generator=gen).to(torch.bfloat16)
    q = torch.randn(B, H, d_h, device="cuda", generator=gen).to(torch.bfloat16)
    lens = torch.full((B,), T, dtype=torch.int32, device="cuda")
    got = from_dev(L.lrkv_mha_decode(k, v, lens, T, q))
    for b, h in ((0, 0), (17, 31), (31, 5)):
        kk = k[b, :, h].float().cpu().numpy().astype(np.float64)
        vv = v[b, :, h].float().cpu().numpy().astype(np.float64)
        qq = q[b, h].float().cpu().numpy().astype(np.float64)
        want = O.softmax_attention(qq, kk, vv, 1.0 / np.sqrt(d_h))
        assert err_ratio(got[b, h], want) <= TOL["bf16"], (b, h)


def test_mha_decode_lengths_clamped_to_max_len():
    # lengths above max_len (and negative ones) are clamped to [0, max_len]
    say("case mha max_len clamp")
    T = 400
    d = mha_inputs(batch=3, capacity=T, heads=8, head_dim=128, lens=[400, 250, 100], dtype="bf16", seed=12)
    lens = torch.tensor([400, 250, -5], dtype=torch.int32, device="cuda")
    dt = d["dtype"]
    got = from_dev(L.lrkv_mha_decode(to_dev(d["k"], dt), to_dev(d["v"], dt), lens, 300, to_dev(d["q"], dt)))
    clamped = dict(d, seq_lens=np.array([300, 250, 0], np.int32))
    want = oracle_mha(clamped)
    assert err_ratio(got, want) <= TOL[dt]
    assert np.all(got[2] == 0)
