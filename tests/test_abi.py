"""C-ABI surface on the host: the library loads, exports every entry point the
header declares, and rejects invalid arguments before launching anything.

No case here reaches a kernel launch: each one fails host validation (the
pointers are fake, aligned or not, and are never dereferenced).  The error
cases are skipped where a GPU is visible, so a validation bug can never turn
a fake pointer into a launch on a real device.
"""
import ctypes
import os
import re

import pytest
import torch

import rank_compressed_kv_lrkv_amd as L
from rank_compressed_kv_lrkv_amd import binding as Bd

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "lrkv.h")
F32, BF16 = 0, 1
OK, NULL, SHAPE, DTYPE, ALIGN, CAP, WS = 0, 1, 2, 3, 4, 5, 6

no_gpu = pytest.mark.skipif(torch.cuda.is_available(), reason="host-validation cases use fake device pointers")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lrkv_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = L.library()
    names = declared_functions()
    assert set(names) == set(Bd.EXPORTED), names
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_elem_count():
    assert L.lrkv_status_string(0) == "ok"
    for s in range(1, 9):
        assert L.lrkv_status_string(s) not in ("ok", "unknown status")
    assert L.lrkv_status_string(99) == "unknown status"
    assert L.lrkv_cache_elems_per_token(32, 128, 16) == 2 * (128 + 32 * 16)
    assert L.lrkv_cache_elems_per_token(18, 128, 55) == 2236
    assert L.lrkv_cache_elems_per_token(4, 16, 0) == 32
    assert L.lrkv_cache_elems_per_token(0, 16, 4) == -1
    assert L.lrkv_cache_elems_per_token(4, 16, -1) == -1


def test_decode_scan_kernel_names():
    lib = L.library()
    assert lib.lrkv_decode_scan_kernel(BF16, 32, 128, 16) == b"decode_mfma_kernel"
    assert lib.lrkv_decode_scan_kernel(BF16, 64, 64, 32) == b"decode_mfma_kernel"
    assert lib.lrkv_decode_scan_kernel(BF16, 32, 128, 0) == b"decode_mfma_kernel"
    assert lib.lrkv_decode_scan_kernel(BF16, 8, 64, 8) == b"decode_split_kernel"     # heads not a multiple of 32
    assert lib.lrkv_decode_scan_kernel(BF16, 32, 32, 16) == b"decode_split_kernel"   # head_dim 32
    assert lib.lrkv_decode_scan_kernel(BF16, 32, 128, 64) == b"decode_split_kernel"  # rank 64
    assert lib.lrkv_decode_scan_kernel(F32, 32, 128, 16) == b"decode_split_kernel"   # fp32 storage
    assert lib.lrkv_decode_scan_kernel(BF16, 32, 128, 54) == b"decode_mfma_any_kernel"  # the pages' ranks
    assert lib.lrkv_decode_scan_kernel(BF16, 18, 128, 55) == b"decode_mfma_any_kernel"
    assert lib.lrkv_decode_scan_kernel(BF16, 12, 128, 51) == b"decode_mfma_any_kernel"
    assert lib.lrkv_decode_scan_kernel(BF16, 6, 128, 128) == b"decode_mfma_any_kernel"  # four column copies
    assert lib.lrkv_decode_scan_kernel(BF16, 20, 128, 128) == b"decode_generic_kernel"  # 32-word windows, < 32 heads
    assert lib.lrkv_decode_scan_kernel(BF16, 32, 128, 128) == b"decode_mfma_any_kernel"
    assert lib.lrkv_decode_scan_kernel(BF16, 6, 128, 112) == b"decode_mfma_any_kernel"
    assert lib.lrkv_decode_scan_kernel(F32, 6, 128, 128) == b"decode_generic_kernel"
    assert lib.lrkv_decode_scan_kernel(BF16, 7, 128, 55) == b"decode_generic_kernel"   # heads * rank odd
    assert lib.lrkv_decode_scan_kernel(BF16, 32, 128, 7) == b"decode_generic_kernel"   # rank below 8
    assert lib.lrkv_decode_scan_kernel(BF16, 32, 64, 54) == b"decode_generic_kernel"   # head_dim 64
    assert lib.lrkv_decode_scan_kernel(BF16, 8, 64, 4) == b"decode_generic_kernel"    # bf16 rank 4
    assert lib.lrkv_decode_scan_kernel(BF16, 96, 64, 8) == b"decode_generic_kernel"   # more than 64 heads
    assert lib.lrkv_decode_scan_kernel(BF16, 32, 128, 129) is None
    assert lib.lrkv_decode_scan_kernel(BF16, 1025, 128, 8) is None
    assert lib.lrkv_decode_scan_kernel(BF16, 32, 24, 16) is None                     # unsupported head_dim
    assert lib.lrkv_decode_scan_kernel(7, 32, 128, 16) is None
    assert L.lrkv_decode_scan_kernel(torch.bfloat16, 32, 128, 16) == "decode_mfma_kernel"


def ws_size(dtype=BF16, B=2, H=8, d_h=64, r=8, cap=256, max_len=256, split=0):
    n = ctypes.c_size_t(0)
    st = L.library().lrkv_decode_workspace_size(dtype, B, H, d_h, r, cap, max_len, split, ctypes.byref(n))
    return st, n.value


def test_workspace_size_formula_any_rank():
    # the any-rank scans keep one partial state per (split, head); the MFMA one (the default
    # for bf16 at head_dim 128) also the absorbed queries, batch * heads * rank fp32
    pad = lambda x: -(-x // 256) * 256
    for dt, qt in ((F32, 0), (BF16, pad(2 * 18 * 55 * 4))):
        st, n = ws_size(dt, B=2, H=18, d_h=128, r=55, cap=1024, max_len=1000, split=128)
        assert st == OK
        states = 2 * -(-1000 // 128) * 18
        assert n == pad(states * 2 * 4) + pad(states * (128 + 55) * 4) + qt, dt


def test_workspace_size_formula():
    # partial states: B * partials * H * (2 + d_h + r) fp32, each part padded to 256 bytes
    st, n = ws_size(BF16, B=2, H=8, d_h=64, r=8, cap=1024, max_len=1000, split=128)
    assert st == OK
    n_splits = -(-1000 // 128)
    slots = 256 // (8 * 8)
    states = 2 * n_splits * slots * 8
    pad = lambda x: -(-x // 256) * 256
    assert n == pad(states * 2 * 4) + pad(states * (64 + 8) * 4)


@pytest.mark.parametrize("kw,want", [
    (dict(dtype=2), DTYPE),
    (dict(H=0), SHAPE), (dict(d_h=0), SHAPE), (dict(r=-1), SHAPE), (dict(cap=0), SHAPE),
    (dict(d_h=24), SHAPE),                       # unsupported head width
    (dict(r=129), SHAPE),                        # rank beyond the any-rank scan's 128
    (dict(H=1025), SHAPE),                       # heads beyond the any-rank scan's 1024
    (dict(max_len=257), CAP), (dict(max_len=-1), SHAPE),
    (dict(split=100), SHAPE),                    # not a multiple of 64
])
def test_workspace_size_rejects(kw, want):
    assert ws_size(**kw)[0] == want


def test_workspace_size_split_offset_range():
    # one split's latents are addressed through 32-bit offsets: 64 heads x rank 64 x 4 bytes
    # = 16 KiB per token, so 262144-token splits (4 GiB) are rejected and 262080 accepted
    big = dict(dtype=F32, B=1, H=64, d_h=128, r=64, cap=262144, max_len=262144)
    assert ws_size(**big, split=262144)[0] == SHAPE
    assert ws_size(**big, split=262080)[0] == OK


def test_workspace_size_null_out():
    assert L.library().lrkv_decode_workspace_size(BF16, 1, 4, 64, 8, 64, 64, 0, None) == NULL


FAKE = 0x100000           # aligned, never dereferenced
MIS = 0x100008            # 8-byte aligned only


def decode_call(**over):
    a = dict(dtype=BF16, B=2, H=8, d_h=64, r=8, cap=256, k=FAKE, v=FAKE, zk=FAKE, zv=FAKE, lens=FAKE,
             max_len=256, q=FAKE, bk=FAKE, bv=FAKE, scale=0.0, split=0, out=FAKE, ws=FAKE, ws_bytes=1 << 30)
    a.update(over)
    return L.library().lrkv_decode(a["dtype"], a["B"], a["H"], a["d_h"], a["r"], a["cap"], a["k"], a["v"],
                                   a["zk"], a["zv"], a["lens"], a["max_len"], a["q"], a["bk"], a["bv"],
                                   a["scale"], a["split"], a["out"], a["ws"], a["ws_bytes"], None)


@no_gpu
@pytest.mark.parametrize("kw,want", [
    (dict(k=None), NULL), (dict(v=None), NULL), (dict(zk=None), NULL), (dict(zv=None), NULL),
    (dict(lens=None), NULL), (dict(q=None), NULL), (dict(bk=None), NULL), (dict(bv=None), NULL),
    (dict(out=None), NULL),
    (dict(ws=None), WS), (dict(ws_bytes=16), WS),
    (dict(k=MIS), ALIGN), (dict(zv=MIS), ALIGN), (dict(q=MIS), ALIGN), (dict(out=MIS), ALIGN),
    (dict(ws=MIS), ALIGN), (dict(lens=FAKE + 2), ALIGN),
    (dict(max_len=300), CAP), (dict(dtype=7), DTYPE), (dict(d_h=40), SHAPE),
    (dict(split=96), SHAPE),
])
def test_decode_rejects_before_launch(kw, want):
    assert decode_call(**kw) == want


@no_gpu
def test_decode_empty_batch_is_noop():
    assert decode_call(B=0, k=None, v=None, q=None, out=None, ws=None) == OK


def append_call(**over):
    a = dict(dtype=BF16, B=2, H=8, d_h=64, r=8, cap=256, k=FAKE, v=FAKE, zk=FAKE, zv=FAKE, pos=FAKE, n=4,
             nk=FAKE, nv=FAKE, nzk=FAKE, nzv=FAKE)
    a.update(over)
    return L.library().lrkv_append(a["dtype"], a["B"], a["H"], a["d_h"], a["r"], a["cap"], a["k"], a["v"],
                                   a["zk"], a["zv"], a["pos"], a["n"], a["nk"], a["nv"], a["nzk"], a["nzv"],
                                   None)


@no_gpu
@pytest.mark.parametrize("kw,want", [
    (dict(k=None), NULL), (dict(pos=None), NULL), (dict(nzk=None), NULL),
    (dict(nk=MIS), ALIGN), (dict(zk=MIS), ALIGN), (dict(pos=FAKE + 1), ALIGN),
    (dict(n=-1), SHAPE), (dict(d_h=20), SHAPE), (dict(dtype=5), DTYPE), (dict(cap=0), SHAPE),
])
def test_append_rejects_before_launch(kw, want):
    assert append_call(**kw) == want


@no_gpu
def test_append_zero_rows_is_noop():
    assert append_call(n=0, k=None, v=None, pos=None, nk=None, nv=None) == OK


@no_gpu
def test_prefill_kernel_names():
    """bf16 at ranks 0/8/16/32 and head_dim 64/128 runs on MFMA, at the
    other ranks up to 128 on its windowed form where the windows fit; fp32 and the other ranks up to 128 on
    the vector-ALU kernel; larger shapes on neither."""
    assert L.lrkv_prefill_kernel(torch.bfloat16, 32, 128, 16) == "prefill_kernel"
    assert L.lrkv_prefill_kernel(torch.bfloat16, 4, 64, 0) == "prefill_kernel"
    assert L.lrkv_prefill_kernel(torch.bfloat16, 32, 128, 54) == "prefill_wide_kernel"
    assert L.lrkv_prefill_kernel(torch.bfloat16, 12, 64, 46) == "prefill_wide_kernel"
    assert L.lrkv_prefill_kernel(torch.bfloat16, 12, 128, 51) == "prefill_wide_kernel"      # odd rank, even heads
    assert L.lrkv_prefill_kernel(torch.bfloat16, 9, 128, 55) == "prefill_generic_kernel"    # odd heads x odd rank
    assert L.lrkv_prefill_kernel(torch.bfloat16, 12, 32, 54) == "prefill_generic_kernel"    # head_dim 32
    assert L.lrkv_prefill_kernel(torch.bfloat16, 6, 128, 128) == "prefill_wide_kernel"
    assert L.lrkv_prefill_kernel(torch.bfloat16, 6, 128, 127) == "prefill_generic_kernel"   # window past 128
    assert L.lrkv_prefill_kernel(torch.float32, 32, 128, 16) == "prefill_generic_kernel"
    assert L.lrkv_prefill_kernel(torch.float32, 3, 16, 5) == "prefill_generic_kernel"
    assert L.lrkv_prefill_kernel(torch.bfloat16, 32, 128, 129) is None
    assert L.lrkv_prefill_kernel(torch.bfloat16, 32, 256, 16) is None
    assert L.lrkv_prefill_kernel(torch.float32, 70000, 128, 16) is None   # grid limit of the vector-ALU kernel


def prefill_call(**over):
    a = dict(dtype=BF16, B=1, H=8, d_h=64, r=8, cap=128, k=None, v=None, zk=None, zv=None, L=64, q=FAKE,
             ks=FAKE, vs=FAKE, zkn=FAKE, zvn=FAKE, bk=FAKE, bv=FAKE, scale=0.0, out=FAKE)
    a.update(over)
    return L.library().lrkv_prefill(a["dtype"], a["B"], a["H"], a["d_h"], a["r"], a["cap"], a["k"], a["v"],
                                    a["zk"], a["zv"], a["L"], a["q"], a["ks"], a["vs"], a["zkn"], a["zvn"],
                                    a["bk"], a["bv"], a["scale"], a["out"], None)


@no_gpu
@pytest.mark.parametrize("kw,want", [
    (dict(r=130), SHAPE),                        # rank above 128: neither prefill kernel
    (dict(d_h=256, r=16), SHAPE),                # head_dim above 128
    (dict(L=-1), SHAPE),
    (dict(k=FAKE), NULL),                        # cache pointers: all or none
    (dict(k=FAKE, v=FAKE, zk=FAKE, zv=FAKE, L=256), CAP),
])
def test_prefill_rejects_before_launch(kw, want):
    assert prefill_call(**kw) == want


def chunk_call(**over):
    a = dict(dtype=BF16, B=2, H=8, d_h=64, r=8, cap=256, k=FAKE, v=FAKE, zk=FAKE, zv=FAKE, start=FAKE, max_start=100,
             n=64, q=FAKE, ks=FAKE, vs=FAKE, zkn=FAKE, zvn=FAKE, bk=FAKE, bv=FAKE, scale=0.0, out=FAKE)
    a.update(over)
    return L.library().lrkv_prefill_chunk(a["dtype"], a["B"], a["H"], a["d_h"], a["r"], a["cap"], a["k"], a["v"],
                                          a["zk"], a["zv"], a["start"], a["max_start"], a["n"], a["q"], a["ks"],
                                          a["vs"], a["zkn"], a["zvn"], a["bk"], a["bv"], a["scale"], a["out"], None)


@no_gpu
@pytest.mark.parametrize("kw,want", [
    (dict(r=130), SHAPE),                        # rank above 128: neither prefill kernel
    (dict(d_h=256), SHAPE),                      # head_dim above 128
    (dict(max_start=-1), SHAPE), (dict(n=-1), SHAPE),
    (dict(max_start=200, n=64), CAP),            # history bound + new tokens past the capacity
    (dict(k=None), NULL), (dict(start=None), NULL), (dict(q=None), NULL), (dict(bk=None), NULL),
    (dict(start=FAKE + 2), ALIGN), (dict(zv=MIS), ALIGN), (dict(ks=MIS), ALIGN),
])
def test_prefill_chunk_rejects_before_launch(kw, want):
    assert chunk_call(**kw) == want


@no_gpu
def test_prefill_chunk_empty_is_noop():
    assert chunk_call(n=0, k=None, q=None, out=None) == OK



def project_call(**over):
    a = dict(dtype=BF16, B=2, H=8, d_h=64, r=8, cap=256, k=FAKE, v=FAKE, zk=FAKE, zv=FAKE, pos=FAKE, n=16, d=512,
             x=FAKE, w=FAKE, ws=None, ws_bytes=0)
    a.update(over)
    return L.library().lrkv_project_append(a["dtype"], a["B"], a["H"], a["d_h"], a["r"], a["cap"], a["k"], a["v"],
                                           a["zk"], a["zv"], a["pos"], a["n"], a["d"], a["x"], a["w"], a["ws"],
                                           a["ws_bytes"], None)


@no_gpu
@pytest.mark.parametrize("kw,want", [
    (dict(dtype=7), DTYPE), (dict(n=-1), SHAPE), (dict(d=0), SHAPE), (dict(d=65537), SHAPE),
    (dict(d_h=20), SHAPE), (dict(cap=0), SHAPE),
    (dict(x=None), NULL), (dict(w=None), NULL), (dict(pos=None), NULL), (dict(zv=None), NULL),
    (dict(x=MIS), ALIGN), (dict(w=MIS), ALIGN), (dict(pos=FAKE + 2), ALIGN), (dict(zk=MIS), ALIGN),
    (dict(ws=MIS, ws_bytes=1 << 20), ALIGN),
])
def test_project_append_rejects_before_launch(kw, want):
    assert project_call(**kw) == want


@no_gpu
def test_project_append_empty_is_noop():
    assert project_call(n=0, x=None, k=None, pos=None) == OK
    assert project_call(B=0, x=None, w=None) == OK


def pack_call(**over):
    a = dict(dtype=BF16, H=8, d_h=64, r=8, d=512, wk=FAKE, wv=FAKE, uk=FAKE, uv=FAKE, out=FAKE)
    a.update(over)
    return L.library().lrkv_pack_projection(a["dtype"], a["H"], a["d_h"], a["r"], a["d"], a["wk"], a["wv"],
                                            a["uk"], a["uv"], a["out"], None)


@no_gpu
@pytest.mark.parametrize("kw,want", [
    (dict(dtype=2), DTYPE), (dict(H=0), SHAPE), (dict(r=-1), SHAPE), (dict(d=-1), SHAPE),
    (dict(wk=None), NULL), (dict(out=None), NULL), (dict(uk=None), NULL),
    (dict(wv=FAKE + 1), ALIGN), (dict(dtype=F32, out=FAKE + 2), ALIGN),
])
def test_pack_projection_rejects_before_launch(kw, want):
    assert pack_call(**kw) == want


@no_gpu
def test_pack_projection_empty_is_noop():
    assert pack_call(d=0, wk=None, out=None) == OK


def test_project_kernel_names():
    # host-only: the choice depends on the sizes, on whether a workspace is
    # given, and on the compute-unit count for the large-tile kernel (256 on
    # MI355X, also the value assumed without a GPU)
    k = lambda *a: L.lrkv_project_kernel(*a)
    bf, f32 = torch.bfloat16, torch.float32
    assert k(f32, 4, 4096, 32, 128, 16, 4096) == "project_append_valu_kernel"
    assert k(bf, 2, 33, 3, 40, 8, 72) == "project_append_valu_kernel"
    assert k(bf, 32, 1, 32, 128, 16, 4096) == "project_splitk_kernel"
    assert k(bf, 32, 1, 32, 128, 16, 4096, False) == "project_skinny_kernel"
    assert k(bf, 8, 8, 32, 128, 16, 4096, False) == "project_skinny_kernel"
    assert k(bf, 2, 130, 32, 128, 16, 4096) == "project_append_kernel"
    assert k(bf, 4, 4096, 32, 128, 16, 4064) == "project_append_kernel"      # d not a multiple of 64
    if not torch.cuda.is_available() or torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert k(bf, 4, 4096, 32, 128, 16, 4096) == "project_gemm_kernel"
    assert k(bf, 0, 4, 32, 128, 16, 4096) is None
    assert k(bf, 4, 4, 32, 128, 16, 0) is None


def test_project_workspace_size():
    # a few tokens: 16 slices of the contraction (at least one 16-wide chunk
    # per wave), one fp32 partial per slice, token and output; else none
    ws = lambda *a: L.lrkv_project_workspace_size(*a)
    bf = torch.bfloat16
    assert ws(bf, 32, 1, 32, 128, 16, 4096) == 16 * 32 * 1280 * 4
    assert ws(bf, 8, 8, 8, 64, 8, 128) == 2 * 64 * 256 * 4          # 8 chunks: 2 slices
    assert ws(bf, 2, 130, 32, 128, 16, 4096) == 0
    assert ws(torch.float32, 1, 4, 4, 16, 4, 64) == 0


def test_mha_workspace_size_formula():
    # [batch][splits][heads] x (m, l) plus [batch][splits][heads][head_dim], fp32
    n = ctypes.c_size_t(0)
    assert L.library().lrkv_mha_decode_workspace_size(BF16, 2, 8, 64, 4096, 1000, 256, ctypes.byref(n)) == OK
    assert n.value == 2 * 4 * 8 * (2 + 64) * 4
    assert L.library().lrkv_mha_decode_workspace_size(BF16, 2, 8, 64, 4096, 0, 256, ctypes.byref(n)) == OK
    assert n.value == 0


def mha_call(**over):
    a = dict(dtype=BF16, B=2, H=8, d_h=128, cap=256, k=FAKE, v=FAKE, lens=FAKE, max_len=200, q=FAKE, scale=0.0,
             split=64, out=FAKE, ws=FAKE, ws_bytes=1 << 20)
    a.update(over)
    return L.library().lrkv_mha_decode(a["dtype"], a["B"], a["H"], a["d_h"], a["cap"], a["k"], a["v"], a["lens"],
                                       a["max_len"], a["q"], a["scale"], a["split"], a["out"], a["ws"],
                                       a["ws_bytes"], None)


@no_gpu
@pytest.mark.parametrize("kw,want", [
    (dict(dtype=4), DTYPE), (dict(d_h=96), SHAPE), (dict(H=0), SHAPE), (dict(split=100), SHAPE),
    (dict(max_len=300), CAP), (dict(k=None), NULL), (dict(lens=None), NULL), (dict(out=None), NULL),
    (dict(ws=None), WS), (dict(ws_bytes=16), WS), (dict(q=MIS), ALIGN), (dict(lens=FAKE + 2), ALIGN),
])
def test_mha_decode_rejects_before_launch(kw, want):
    assert mha_call(**kw) == want


@no_gpu
def test_decode_ex_validation():
    lib = L.library()
    n = ctypes.c_size_t(0)
    # engine 2 (MFMA scan) only on its shapes; engine 1 everywhere the vector scan runs
    assert lib.lrkv_decode_workspace_size_ex(2, BF16, 2, 8, 64, 8, 256, 256, 0, ctypes.byref(n)) == SHAPE
    assert lib.lrkv_decode_workspace_size_ex(1, BF16, 2, 32, 128, 16, 256, 256, 0, ctypes.byref(n)) == OK
    assert lib.lrkv_decode_workspace_size_ex(5, BF16, 2, 32, 128, 16, 256, 256, 0, ctypes.byref(n)) == SHAPE
    assert lib.lrkv_decode_workspace_size_ex(-1, BF16, 2, 32, 128, 16, 256, 256, 0, ctypes.byref(n)) == SHAPE
    # engine 3 (any-rank scan) takes every shape of the envelope; the tuned scans not the pages' odd ranks
    assert lib.lrkv_decode_workspace_size_ex(3, BF16, 2, 32, 128, 16, 256, 256, 0, ctypes.byref(n)) == OK
    assert lib.lrkv_decode_workspace_size_ex(3, F32, 2, 18, 128, 55, 256, 256, 0, ctypes.byref(n)) == OK
    assert lib.lrkv_decode_workspace_size_ex(1, BF16, 2, 18, 128, 55, 256, 256, 0, ctypes.byref(n)) == SHAPE
    assert lib.lrkv_decode_workspace_size_ex(2, BF16, 2, 32, 128, 54, 256, 256, 0, ctypes.byref(n)) == SHAPE
    # engine 4 (any-rank MFMA scan): bf16, head_dim 128, ranks 8..128 with heads * rank even; its
    # workspace adds the absorbed queries (batch * heads * rank fp32) to the partial states
    assert lib.lrkv_decode_workspace_size_ex(4, BF16, 2, 32, 128, 16, 256, 256, 0, ctypes.byref(n)) == OK
    assert lib.lrkv_decode_workspace_size_ex(4, F32, 2, 32, 128, 54, 256, 256, 0, ctypes.byref(n)) == SHAPE
    assert lib.lrkv_decode_workspace_size_ex(4, BF16, 2, 32, 64, 54, 256, 256, 0, ctypes.byref(n)) == SHAPE
    assert lib.lrkv_decode_workspace_size_ex(4, BF16, 2, 7, 128, 55, 256, 256, 0, ctypes.byref(n)) == SHAPE
    assert lib.lrkv_decode_workspace_size_ex(4, BF16, 2, 32, 128, 7, 256, 256, 0, ctypes.byref(n)) == SHAPE
    assert lib.lrkv_decode_workspace_size_ex(4, BF16, 2, 32, 128, 129, 256, 256, 0, ctypes.byref(n)) == SHAPE
    w3, w4 = ctypes.c_size_t(0), ctypes.c_size_t(0)
    assert lib.lrkv_decode_workspace_size_ex(3, BF16, 2, 32, 128, 54, 256, 256, 128, ctypes.byref(w3)) == OK
    assert lib.lrkv_decode_workspace_size_ex(4, BF16, 2, 32, 128, 54, 256, 256, 128, ctypes.byref(w4)) == OK
    assert w4.value == w3.value + (2 * 32 * 54 * 4 + 255) // 256 * 256
    # the default engine matches lrkv_decode_workspace_size
    m = ctypes.c_size_t(0)
    assert lib.lrkv_decode_workspace_size_ex(0, BF16, 2, 32, 128, 16, 256, 256, 0, ctypes.byref(n)) == OK
    assert lib.lrkv_decode_workspace_size(BF16, 2, 32, 128, 16, 256, 256, 0, ctypes.byref(m)) == OK
    assert n.value == m.value
    p = 16
    for phases in (0, 4, -1):
        st = lib.lrkv_decode_ex(1, phases, BF16, 2, 32, 128, 16, 256, p, p, p, p, p, 256, p, p, p,
                                ctypes.c_float(0.0), 0, p, p, 1 << 30, None)
        assert st == SHAPE, (phases, st)


def train_bwd_call(**over):
    a = dict(dtype=BF16, B=1, H=8, d_h=64, r=8, L=64, q=FAKE, ks=FAKE, vs=FAKE, zk=FAKE, zv=FAKE, bk=FAKE, bv=FAKE,
             out=FAKE, lse=FAKE, dout=FAKE, scale=0.0, dq=FAKE, dks=FAKE, dvs=FAKE, dzk=FAKE, dzv=FAKE, dbk=FAKE,
             dbv=FAKE, ws=FAKE, wsb=1 << 30)
    a.update(over)
    return L.library().lrkv_train_backward(
        a["dtype"], a["B"], a["H"], a["d_h"], a["r"], a["L"], a["q"], a["ks"], a["vs"], a["zk"], a["zv"], a["bk"],
        a["bv"], a["out"], a["lse"], a["dout"], a["scale"], a["dq"], a["dks"], a["dvs"], a["dzk"], a["dzv"], a["dbk"],
        a["dbv"], a["ws"], a["wsb"], None)


def test_train_workspace_size():
    lib = L.library()
    n = ctypes.c_size_t(0)
    assert lib.lrkv_train_backward_workspace_size(BF16, 4, 32, 128, 16, 4096, ctypes.byref(n)) == OK
    al = lambda x: (x + 255) // 256 * 256
    B, H, D, R, Lq = 4, 32, 128, 16, 4096
    nb, nkb = (Lq + 31) // 32, (Lq + 127) // 128       # 32-token query blocks, 128-token key blocks
    # Q B^K and dO B^V (bf16), lse and D per padded row, per-head dK_h and
    # dV_h, per-key-block dB^K and dB^V
    want = 2 * al(B * Lq * H * R * 2) + 2 * al(B * H * nb * 32 * 4) + 2 * al(H * B * Lq * D * 4) + \
        2 * al(B * nkb * H * D * R * 4)
    assert n.value == want
    assert lib.lrkv_train_backward_workspace_size(BF16, 4, 30, 128, 16, 4096, ctypes.byref(n)) == SHAPE
    assert lib.lrkv_train_backward_workspace_size(F32, 4, 32, 128, 16, 4096, ctypes.byref(n)) == SHAPE
    assert lib.lrkv_train_backward_workspace_size(BF16, 4, 32, 96, 16, 4096, ctypes.byref(n)) == SHAPE
    assert lib.lrkv_train_backward_workspace_size(BF16, 4, 32, 128, 24, 4096, ctypes.byref(n)) == SHAPE
    assert lib.lrkv_train_backward_workspace_size(BF16, 4, 32, 128, 16, -1, ctypes.byref(n)) == SHAPE
    assert lib.lrkv_train_backward_workspace_size(BF16, 4, 32, 128, 16, 4096, None) == NULL


@no_gpu
@pytest.mark.parametrize("kw,want", [
    (dict(dtype=F32), SHAPE), (dict(dtype=7), DTYPE), (dict(H=6), SHAPE), (dict(d_h=32), SHAPE),
    (dict(r=4), SHAPE), (dict(L=-1), SHAPE), (dict(B=1 << 20, L=1 << 12), SHAPE),
    (dict(q=None), NULL), (dict(lse=None), NULL), (dict(dout=None), NULL), (dict(dbk=None), NULL),
    (dict(dzv=None), NULL), (dict(ws=None), NULL), (dict(wsb=1024), WS),
    (dict(q=MIS), ALIGN), (dict(dq=FAKE + 4), ALIGN), (dict(dks=FAKE + 2), ALIGN), (dict(ws=MIS), ALIGN),
])
def test_train_backward_rejects_before_launch(kw, want):
    assert train_bwd_call(**kw) == want


@no_gpu
def test_train_forward_rejects_before_launch():
    lib = L.library()
    call = lambda **o: lib.lrkv_train_forward(
        o.get("dtype", BF16), 1, o.get("H", 8), 64, 8, o.get("L", 64), o.get("q", FAKE), FAKE, FAKE, FAKE, FAKE,
        FAKE, FAKE, ctypes.c_float(0.0), FAKE, o.get("lse", FAKE), None)
    assert call(dtype=F32) == SHAPE
    assert call(H=6) == SHAPE
    assert call(L=-1) == SHAPE
    assert call(lse=None) == NULL
    assert call(q=MIS) == ALIGN
    assert call(lse=FAKE + 2) == ALIGN
    assert call(L=0, q=None, lse=None) == OK
