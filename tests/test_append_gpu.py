"""lrkv_append (HIP, through the C ABI): bit-exact copies at per-sequence
offsets, nothing else touched, rows outside the cache dropped."""
import numpy as np
import pytest
import torch

import oracle as O
import rank_compressed_kv_lrkv_amd as L
from rank_compressed_kv_lrkv_amd.workloads import append_inputs, DECODE_WORKLOADS, decode_inputs
from tests.gpu_util import check_decode_after_append, device_cache, say, to_dev

pytestmark = pytest.mark.gpu


def host_bits(t):
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy()
    return t.view(torch.int32).cpu().numpy()


def stored_bits(a, dtype):
    return np.ascontiguousarray(a).view(np.int16 if dtype == "bf16" else np.int32)


@pytest.mark.parametrize("dt,H,d_h,r", [("bf16", 8, 64, 8), ("bf16", 32, 128, 16), ("f32", 4, 16, 4),
                                         ("bf16", 4, 32, 0)])
def test_append_bit_exact(dt, H, d_h, r):
    B, T, n = 3, 40, 7
    say(f"case append {dt} H={H} d_h={d_h} r={r}")
    rng = np.random.default_rng(17)
    base = decode_inputs(DECODE_WORKLOADS["small_bf16_T2k"].__class__("canary", B, H, d_h, r, T, dt, 99))
    new = append_inputs(B, n, H, d_h, r, dt, seed=int(rng.integers(1 << 30)))
    cache = device_cache(base)
    pos = np.array([0, 13, T - n], np.int32)
    L.lrkv_append(cache, torch.from_numpy(pos).cuda(), *(to_dev(new[k], dt) for k in ("k_s", "v_s", "z_k", "z_v")))
    torch.cuda.synchronize()
    want = O.append({k: base[k] for k in ("k_s", "v_s", "z_k", "z_v")}, pos, new)
    for k, t in (("k_s", cache.k_s), ("v_s", cache.v_s), ("z_k", cache.z_k), ("z_v", cache.z_v)):
        assert np.array_equal(host_bits(t), stored_bits(want[k], dt)), k


def test_append_drops_rows_outside_cache():
    dt, B, H, d_h, r, T, n = "bf16", 2, 4, 32, 8, 16, 5
    say("case append out-of-range rows")
    base = decode_inputs(DECODE_WORKLOADS["small_bf16_T2k"].__class__("canary", B, H, d_h, r, T, dt, 5))
    new = append_inputs(B, n, H, d_h, r, dt, seed=6)
    cache = device_cache(base)
    pos = np.array([T - 2, -3], np.int32)          # rows at slots >= T or < 0 are dropped
    L.lrkv_append(cache, torch.from_numpy(pos).cuda(), *(to_dev(new[k], dt) for k in ("k_s", "v_s", "z_k", "z_v")))
    torch.cuda.synchronize()
    for k, t in (("k_s", cache.k_s), ("z_v", cache.z_v)):
        got = host_bits(t)
        want = stored_bits(base[k], dt).copy()
        nb = stored_bits(new[k], dt)
        want[0, T - 2:T] = nb[0, :2]
        want[1, 0:2] = nb[1, 3:5]
        assert np.array_equal(got, want), k


def test_decode_after_incremental_appends():
    say("case decode after appends")
    check_decode_after_append()
