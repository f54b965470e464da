"""The entry points captured in a HIP graph (torch.cuda.CUDAGraph; the
binding passes torch's current stream, which is the capture stream inside
torch.cuda.graph) and replayed.

The library allocates nothing, synchronises nothing and clears no memory
with memset, so a serving loop may capture its launches once and replay
them.  Each test captures one step, replays it several times with eager work
between the replays (new inputs copied into the captured tensors, unrelated
kernels, host synchronisations), and checks every replay bit for bit
against the same calls made eagerly on the same inputs into a second set of
buffers; the decode step and the prefill are also checked against the
float64 oracle.
"""
import numpy as np
import pytest
import torch

import oracle as O
import rank_compressed_kv_lrkv_amd as L
from rank_compressed_kv_lrkv_amd.workloads import DecodeWorkload, _store, as_f64, decode_inputs, prefill_inputs, \
    PrefillWorkload, projection_inputs
from tests.gpu_util import TOL, device_cache, err_ratio, from_dev, oracle_decode, say, to_dev

pytestmark = pytest.mark.gpu
KEYS = ("k_s", "v_s", "z_k", "z_v")
TORCH_DT = {"bf16": torch.bfloat16, "f32": torch.float32}
REPLAYS = 4


def bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


def same(a, b):
    return torch.equal(bits(a), bits(b))


def clone_cache(c):
    return L.LrkvCache(*(getattr(c, k).clone() for k in KEYS))


def busy_work():
    """Unrelated eager kernels between replays."""
    x = torch.randn(512, 512, device="cuda")
    return float((x @ x).sum())


@pytest.mark.parametrize("name,B,H,d_h,r,T,dt", [
    ("mfma_scan", 2, 32, 128, 16, 512, "bf16"),   # the MFMA scan head shape
    ("split_scan", 3, 8, 64, 8, 300, "bf16"),     # the vector-ALU split scan
    ("f32", 2, 4, 16, 4, 96, "f32"),
])
def test_append_decode_step_graph(name, B, H, d_h, r, T, dt):
    """One decode step, append the new token's rows at pos[b] then decode
    over pos[b] + 1 tokens, captured once and replayed REPLAYS times."""
    say(f"case graph decode step {name} B={B} H={H} d_h={d_h} r={r} T={T} {dt}")
    lens0 = np.array([T - REPLAYS - 3, T // 3, 1][:B], np.int32)
    d = decode_inputs(DecodeWorkload("graph_" + name, B, H, d_h, r, T, dt, 515), lens=lens0)
    say(f"  scan kernel {L.lrkv_decode_scan_kernel(TORCH_DT[dt], H, d_h, r)}")
    cache = device_cache(d)
    ref = clone_cache(cache)
    tdt = TORCH_DT[dt]
    q = torch.empty(B, H, d_h, dtype=tdt, device="cuda")
    rows = {"k_s": torch.empty(B, 1, d_h, dtype=tdt, device="cuda"),
            "v_s": torch.empty(B, 1, d_h, dtype=tdt, device="cuda"),
            "z_k": torch.empty(B, 1, H, r, dtype=tdt, device="cuda"),
            "z_v": torch.empty(B, 1, H, r, dtype=tdt, device="cuda")}
    pos = torch.zeros(B, dtype=torch.int32, device="cuda")
    lens = torch.ones(B, dtype=torch.int32, device="cuda")
    b_k, b_v = to_dev(d["b_k"], dt), to_dev(d["b_v"], dt)
    out = torch.empty(B, H, d_h, dtype=tdt, device="cuda")
    ws = L.decode_workspace(cache, T)
    out_ref = torch.empty_like(out)
    ws_ref = L.decode_workspace(ref, T)

    def step(c, o, w):
        L.lrkv_append(c, pos, rows["k_s"], rows["v_s"], rows["z_k"], rows["z_v"])
        L.lrkv_decode(c, lens, T, q, b_k, b_v, out=o, workspace=w)

    # host copy of the logical cache: the rows appended below are written into it
    host = {k: d[k].copy() for k in KEYS}
    rng = np.random.default_rng(99)
    cur = lens0.copy()

    def draw():
        host["q"] = _store(rng.standard_normal((B, H, d_h), dtype=np.float32), dt)
        q.copy_(to_dev(host["q"], dt))
        for k in KEYS:
            new = _store(rng.standard_normal(tuple(rows[k].shape), dtype=np.float32), dt)
            rows[k].copy_(to_dev(new, dt))
            for b in range(B):
                host[k][b, cur[b]] = new[b, 0]
        pos.copy_(torch.from_numpy(cur.copy()))
        lens.copy_(torch.from_numpy(cur + 1))

    # warm up on a side stream (first calls set kernel attributes), then capture
    draw()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        warm = clone_cache(cache)
        step(warm, torch.empty_like(out), L.decode_workspace(warm, T))
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    del warm
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(cache, out, ws)
    torch.cuda.synchronize()

    for i in range(REPLAYS):
        if i:
            draw()
        busy_work()
        g.replay()
        torch.cuda.synchronize()
        step(ref, out_ref, ws_ref)
        torch.cuda.synchronize()
        say(f"  replay {i}: lens {list(cur + 1)}")
        assert same(out, out_ref), f"replay {i}: output differs from the eager call"
        for k in KEYS:
            assert same(getattr(cache, k), getattr(ref, k)), f"replay {i}: cache {k} differs from the eager call"
        cur = cur + 1
        busy_work()
    # the last replay against the oracle, on the host's copy of the cache
    dd = dict(d)
    dd.update(host)
    dd["seq_lens"] = cur.copy()
    e = err_ratio(from_dev(out), oracle_decode(dd))
    say(f"  last replay vs oracle: err/||out||inf = {e:.3e}")
    assert e <= TOL[dt]


def test_prefill_graph():
    B, Lq, H, d_h, r = 2, 200, 8, 128, 16
    say(f"case graph prefill B={B} L={Lq} H={H} d_h={d_h} r={r}")
    d = prefill_inputs(PrefillWorkload("graph_prefill", B, Lq, H, d_h, r, "bf16", 616))
    t = {k: to_dev(d[k], "bf16") for k in ("q",) + KEYS + ("b_k", "b_v")}
    out = torch.empty_like(t["q"])
    out_ref = torch.empty_like(out)
    call = lambda o: L.lrkv_prefill(t["q"], t["k_s"], t["v_s"], t["z_k"], t["z_v"], t["b_k"], t["b_v"], out=o)
    call(out_ref)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out)
    rng = np.random.default_rng(17)
    q_host = d["q"]
    for i in range(REPLAYS):
        if i:
            q_host = _store(rng.standard_normal(d["q"].shape, dtype=np.float32), "bf16")
            t["q"].copy_(to_dev(q_host, "bf16"))
        busy_work()
        g.replay()
        torch.cuda.synchronize()
        call(out_ref)
        torch.cuda.synchronize()
        say(f"  replay {i}")
        assert same(out, out_ref), f"replay {i}: output differs from the eager call"
    f = lambda k: as_f64(d[k], "bf16")
    want = O.prefill(as_f64(q_host, "bf16"), f("k_s"), f("v_s"), f("z_k"), f("z_v"), f("b_k"), f("b_v"))
    e = err_ratio(from_dev(out), want)
    say(f"  last replay vs oracle: err/||out||inf = {e:.3e}")
    assert e <= TOL["bf16"]


@pytest.mark.parametrize("B,n,d,with_ws", [(8, 1, 1024, True), (8, 1, 1024, False), (2, 40, 512, True)])
def test_project_decode_step_graph(B, n, d, with_ws):
    """A serving step from hidden states: the fused projection writes the new
    tokens' cache rows at pos[b], then the decode reads them."""
    H, d_h, r, T, dt = 8, 128, 16, 256, "bf16"
    kernel = L.lrkv_project_kernel(torch.bfloat16, B, n, H, d_h, r, d, with_ws)
    say(f"case graph project+decode B={B} n={n} d={d} workspace={with_ws} kernel={kernel}")
    inp = projection_inputs(batch=B, n_new=n, d_model=d, heads=H, head_dim=d_h, rank=r, dtype=dt, seed=717)
    w = L.lrkv_pack_projection(*(to_dev(inp[k], dt) for k in ("wk", "wv", "uk", "uv")))
    lens0 = np.arange(B, dtype=np.int32) * 7 % (T - n * REPLAYS - 1) + 1
    dec = decode_inputs(DecodeWorkload("graph_proj", B, H, d_h, r, T, dt, 718), lens=lens0)
    cache = device_cache(dec)
    ref = clone_cache(cache)
    x = to_dev(inp["x"], dt)
    q = to_dev(dec["q"], dt)
    b_k, b_v = to_dev(dec["b_k"], dt), to_dev(dec["b_v"], dt)
    pos = torch.from_numpy(lens0.copy()).cuda()
    lens = torch.from_numpy(lens0 + n).cuda()
    nbytes = L.lrkv_project_workspace_size(torch.bfloat16, B, n, H, d_h, r, d) if with_ws else 0
    pws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda") if with_ws else None
    pws_ref = torch.empty_like(pws) if with_ws else None
    out, out_ref = torch.empty_like(q), torch.empty_like(q)
    dws, dws_ref = L.decode_workspace(cache, T), L.decode_workspace(ref, T)

    def step(c, o, pw, dw):
        L.lrkv_project_append(c, pos, x, w, workspace=pw)
        L.lrkv_decode(c, lens, T, q, b_k, b_v, out=o, workspace=dw)

    warm = clone_cache(cache)
    step(warm, torch.empty_like(q), torch.empty_like(pws) if with_ws else None, L.decode_workspace(warm, T))
    torch.cuda.synchronize()
    del warm
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(cache, out, pws, dws)
    rng = np.random.default_rng(5)
    cur = lens0.copy()
    for i in range(REPLAYS):
        if i:
            x.copy_(to_dev(_store(rng.standard_normal(inp["x"].shape, dtype=np.float32), dt), dt))
            pos.copy_(torch.from_numpy(cur.copy()))
            lens.copy_(torch.from_numpy(cur + n))
        busy_work()
        g.replay()
        torch.cuda.synchronize()
        step(ref, out_ref, pws_ref, dws_ref)
        torch.cuda.synchronize()
        say(f"  replay {i}: pos {list(cur[:4])}")
        assert same(out, out_ref), f"replay {i}: output differs from the eager call"
        for k in KEYS:
            assert same(getattr(cache, k), getattr(ref, k)), f"replay {i}: cache {k} differs from the eager call"
        cur = cur + n


CAPTURE_AFTER_INIT = r'''
import sys, torch
import rank_compressed_kv_lrkv_amd as L
torch.cuda.init()
L.lrkv_init()                                   # the only set-up: no eager call before the capture
g0 = torch.Generator(device="cuda").manual_seed(3)
bf = torch.bfloat16
rn = lambda *s, sc=1.0: (torch.randn(*s, device="cuda", generator=g0) * sc).to(bf)
B, Lq, H, D, R, T = 2, 96, 32, 128, 16, 256
q, ks, vs, zk, zv = rn(B, Lq, H, D), rn(B, Lq, D), rn(B, Lq, D), rn(B, Lq, H, R), rn(B, Lq, H, R)
bk, bv, dout = rn(H, D, R, sc=0.25), rn(H, D, R, sc=0.25), rn(B, Lq, H, D)
cache = L.LrkvCache(rn(B, T, D), rn(B, T, D), rn(B, T, H, R), rn(B, T, H, R))
qd = rn(B, H, D)
lens = torch.tensor([T, 77], dtype=torch.int32, device="cuda")
ws = L.decode_workspace(cache, T)
tws = torch.empty(L.lrkv_train_backward_workspace_size(bf, B, H, D, R, Lq), dtype=torch.uint8, device="cuda")
def bufs():
    return dict(po=torch.empty_like(q), do=torch.empty(B, H, D, dtype=bf, device="cuda"),
                to=torch.empty_like(q), lse=torch.empty(B, Lq, H, device="cuda"),
                g={k: torch.empty(s, device="cuda") for k, s in (("dq", (B, Lq, H, D)), ("dk_s", (B, Lq, D)),
                   ("dv_s", (B, Lq, D)), ("dz_k", (B, Lq, H, R)), ("dz_v", (B, Lq, H, R)), ("db_k", (H, D, R)),
                   ("db_v", (H, D, R)))})
def step(o):
    L.lrkv_prefill(q, ks, vs, zk, zv, bk, bv, out=o["po"])
    L.lrkv_decode(cache, lens, T, qd, bk, bv, out=o["do"], workspace=ws)
    L.lrkv_train_forward(q, ks, vs, zk, zv, bk, bv, out=o["to"], lse=o["lse"])
    L.lrkv_train_backward(q, ks, vs, zk, zv, bk, bv, o["to"], o["lse"], dout, workspace=tws, grads=o["g"])
cap, ref = bufs(), bufs()
graph = torch.cuda.CUDAGraph()
with torch.cuda.graph(graph):
    step(cap)
for i in range(3):
    graph.replay()
    torch.cuda.synchronize()
    step(ref)
    torch.cuda.synchronize()
    for k in ("po", "do", "to", "lse"):
        a, b = cap[k], ref[k]
        assert torch.equal(a.view(torch.int16) if a.dtype == bf else a, b.view(torch.int16) if b.dtype == bf else b), (i, k)
    for k in cap["g"]:
        assert torch.equal(cap["g"][k], ref["g"][k]), (i, k)
print("capture after lrkv_init: 3 replays bit-identical to eager calls", flush=True)
'''


def test_capture_after_init_in_a_fresh_process():
    """In a fresh process, lrkv_init and then a capture of prefill, decode
    (MFMA scan) and a training step with no eager call before it: every
    kernel that raises its dynamic-LDS limit at first launch is set up by
    lrkv_init.  Three replays are compared bit for bit with eager calls."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ)
    env["PYTHONPATH"] = root + os.pathsep + env.get("PYTHONPATH", "")
    say("case capture after lrkv_init, fresh process")
    res = subprocess.run([sys.executable, "-c", CAPTURE_AFTER_INIT], cwd=root, env=env, capture_output=True,
                         text=True, timeout=300)
    say(res.stdout.strip()[-2000:])
    assert res.returncode == 0, res.stderr[-4000:]
