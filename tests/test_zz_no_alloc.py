"""lrkv_decode_noalloc (decode with the library's fixed device scratch) against
lrkv_decode with a caller workspace, through the C ABI.

Both run the same scan and merge kernels with the same partition, so their
outputs must agree bit for bit; each is also held to the float64 oracle at
the bf16 bar (2e-2 * ||out||inf).  Two calls in a row, the second with a
smaller input, show that the scratch left by the first call does not leak
into the second.
"""
import ctypes

import numpy as np
import pytest
import torch

import rank_compressed_kv_lrkv_amd as L
from rank_compressed_kv_lrkv_amd.workloads import DECODE_WORKLOADS, decode_inputs
from tests.gpu_util import TOL, device_cache, err_ratio, from_dev, oracle_decode, say, to_dev

pytestmark = pytest.mark.gpu


def both_paths(d, split_tokens=0):
    dt = d["dtype"]
    cache = device_cache(d)
    lens = torch.from_numpy(np.asarray(d["seq_lens"], np.int32)).cuda()
    ml = int(d["capacity"])
    q, bk, bv = to_dev(d["q"], dt), to_dev(d["b_k"], dt), to_dev(d["b_v"], dt)
    out_na = torch.full_like(q, float("nan"))
    L.lrkv_decode_noalloc(cache, lens, ml, q, bk, bv, split_tokens=split_tokens, out=out_na)
    out_ws = L.lrkv_decode(cache, lens, ml, q, bk, bv, split_tokens=split_tokens)
    torch.cuda.synchronize()
    return out_na, out_ws


def check_pair(d, name, split_tokens=0):
    out_na, out_ws = both_paths(d, split_tokens)
    assert torch.equal(out_na.view(torch.int16) if out_na.dtype == torch.bfloat16 else out_na,
                       out_ws.view(torch.int16) if out_ws.dtype == torch.bfloat16 else out_ws), name
    e = err_ratio(from_dev(out_na), oracle_decode(d))
    say(f"  {name}: noalloc == workspace bitwise; err/||out||inf = {e:.3e}")
    assert e <= TOL[d["dtype"]], (name, e)


def test_noalloc_matches_workspace_mfma_scan_then_smaller():
    wl = DECODE_WORKLOADS["mid_bf16_T8k"]
    assert L.lrkv_decode_scan_kernel(torch.bfloat16, wl.heads, wl.head_dim, wl.rank) == "decode_mfma_kernel"
    lens = np.array([1000, 999, 513, 1, 64, 65], np.int32)
    say(f"case noalloc {wl.name} batch=6 capacity=1000 lens={lens.tolist()}")
    check_pair(decode_inputs(wl, batch=6, capacity=1000, lens=lens, seed=31), "mfma scan, first call")
    lens2 = np.array([300, 0], np.int32)
    say(f"case noalloc {wl.name} batch=2 capacity=300 lens={lens2.tolist()}")
    check_pair(decode_inputs(wl, batch=2, capacity=300, lens=lens2, seed=32), "mfma scan, second smaller call")


def test_noalloc_matches_workspace_vector_scan_then_smaller():
    wl = DECODE_WORKLOADS["small_bf16_T2k"]
    assert L.lrkv_decode_scan_kernel(torch.bfloat16, wl.heads, wl.head_dim, wl.rank) == "decode_split_kernel"
    say(f"case noalloc {wl.name} (full size)")
    check_pair(decode_inputs(wl), "vector scan, first call")
    lens2 = np.array([77, 200, 1], np.int32)
    say(f"case noalloc {wl.name} batch=3 capacity=200 lens={lens2.tolist()} split=64")
    check_pair(decode_inputs(wl, batch=3, capacity=200, lens=lens2, seed=33), "vector scan, smaller, split 64",
               split_tokens=64)


def test_noalloc_matches_workspace_any_rank_mfma_then_smaller():
    # the any-rank MFMA scan keeps the absorbed queries in the scratch too
    wl = DECODE_WORKLOADS["rank54_bf16_T8k"]
    assert L.lrkv_decode_scan_kernel(torch.bfloat16, wl.heads, wl.head_dim, wl.rank) == "decode_mfma_any_kernel"
    lens = np.array([1000, 999, 513, 1, 64, 65], np.int32)
    say(f"case noalloc {wl.name} batch=6 capacity=1000 lens={lens.tolist()}")
    check_pair(decode_inputs(wl, batch=6, capacity=1000, lens=lens, seed=34), "any-rank mfma scan, first call")
    lens2 = np.array([300, 0], np.int32)
    say(f"case noalloc {wl.name} batch=2 capacity=300 lens={lens2.tolist()} split=128")
    check_pair(decode_inputs(wl, batch=2, capacity=300, lens=lens2, seed=35), "any-rank mfma scan, smaller",
               split_tokens=128)


def test_noalloc_rejects_requests_beyond_scratch():
    # host validation only: the workspace this fixed split needs (73 MiB) is
    # above the 16 MiB scratch, so the call returns before any launch
    lib = L.library()
    n = ctypes.c_size_t(0)
    assert lib.lrkv_decode_workspace_size(1, 32, 32, 128, 16, 8192, 8192, 64, ctypes.byref(n)) == 0
    assert n.value > 16 << 20
    st = lib.lrkv_decode_noalloc(1, 32, 32, 128, 16, 8192, 16, 16, 16, 16, 16, 8192, 16, 16, 16,
                                 ctypes.c_float(0.0), 64, 16, None)
    assert st == 8, st
    assert L.lrkv_status_string(8) != "unknown status"
