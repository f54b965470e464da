"""ctypes binding of liblrkv: the C entry points under the same names.

Argument marshalling only: every step of the computation runs in the HIP
kernels of liblrkv.so.  Tensors are torch tensors on a ROCm device; their
data pointers and torch's current stream are handed to the library.  There
is no fallback: if the library is missing, or a tensor is not on the GPU,
the call raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass
from typing import Optional

import torch  # imported before the library so both share one HIP runtime

_HERE = os.path.dirname(os.path.abspath(__file__))
# LRKV_LIBRARY names another build of the library (the host-sanitizer build
# of build.py --sanitize, for instance); by default the in-tree one.
LIB_PATH = os.environ.get("LRKV_LIBRARY") or os.path.join(_HERE, "lib", "liblrkv.so")

LRKV_F32 = 0
LRKV_BF16 = 1
STATUS = {0: "LRKV_OK", 1: "LRKV_ERR_NULL", 2: "LRKV_ERR_SHAPE", 3: "LRKV_ERR_DTYPE", 4: "LRKV_ERR_ALIGN",
          5: "LRKV_ERR_CAPACITY", 6: "LRKV_ERR_WORKSPACE", 7: "LRKV_ERR_DEVICE", 8: "LRKV_ERR_SCRATCH"}

EXPORTED = ("lrkv_init", "lrkv_status_string", "lrkv_cache_elems_per_token", "lrkv_append",
            "lrkv_decode_workspace_size", "lrkv_decode_scan_kernel", "lrkv_decode", "lrkv_decode_partial",
            "lrkv_decode_combine", "lrkv_decode_noalloc", "lrkv_decode_workspace_size_ex", "lrkv_decode_ex", "lrkv_prefill_kernel", "lrkv_prefill", "lrkv_prefill_chunk", "lrkv_pack_projection",
            "lrkv_project_kernel", "lrkv_project_workspace_size", "lrkv_project_append",
            "lrkv_mha_decode_workspace_size", "lrkv_mha_decode", "lrkv_train_forward",
            "lrkv_train_backward_workspace_size", "lrkv_train_backward")


class LrkvError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({lrkv_status_string(status)})")


_lib = None

_i32, _i64, _f32, _vp, _sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t


def library() -> ctypes.CDLL:
    """Load liblrkv.so (built in-tree by ``rank_compressed_kv_lrkv_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m rank_compressed_kv_lrkv_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        lib.lrkv_init.argtypes = []
        lib.lrkv_init.restype = _i32
        lib.lrkv_status_string.argtypes = [_i32]
        lib.lrkv_status_string.restype = ctypes.c_char_p
        lib.lrkv_cache_elems_per_token.argtypes = [_i32, _i32, _i32]
        lib.lrkv_cache_elems_per_token.restype = _i64
        lib.lrkv_append.argtypes = [_i32, _i32, _i32, _i32, _i32, _i64, _vp, _vp, _vp, _vp, _vp, _i32,
                                    _vp, _vp, _vp, _vp, _vp]
        lib.lrkv_append.restype = _i32
        lib.lrkv_decode_scan_kernel.argtypes = [_i32, _i32, _i32, _i32]
        lib.lrkv_decode_scan_kernel.restype = ctypes.c_char_p
        lib.lrkv_prefill_kernel.argtypes = [_i32, _i32, _i32, _i32]
        lib.lrkv_prefill_kernel.restype = ctypes.c_char_p
        lib.lrkv_decode_workspace_size.argtypes = [_i32, _i32, _i32, _i32, _i32, _i64, _i64, _i32,
                                                   ctypes.POINTER(_sz)]
        lib.lrkv_decode_workspace_size.restype = _i32
        for fn in (lib.lrkv_decode, lib.lrkv_decode_partial, lib.lrkv_decode_combine):
            fn.argtypes = [_i32, _i32, _i32, _i32, _i32, _i64, _vp, _vp, _vp, _vp, _vp, _i64,
                           _vp, _vp, _vp, _f32, _i32, _vp, _vp, _sz, _vp]
            fn.restype = _i32
        lib.lrkv_decode_workspace_size_ex.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32, _i64, _i64, _i32,
                                                      ctypes.POINTER(_sz)]
        lib.lrkv_decode_workspace_size_ex.restype = _i32
        lib.lrkv_decode_ex.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i64, _vp, _vp, _vp, _vp, _vp, _i64,
                                       _vp, _vp, _vp, _f32, _i32, _vp, _vp, _sz, _vp]
        lib.lrkv_decode_ex.restype = _i32
        lib.lrkv_decode_noalloc.argtypes = [_i32, _i32, _i32, _i32, _i32, _i64, _vp, _vp, _vp, _vp, _vp, _i64,
                                            _vp, _vp, _vp, _f32, _i32, _vp, _vp]
        lib.lrkv_decode_noalloc.restype = _i32
        lib.lrkv_prefill.argtypes = [_i32, _i32, _i32, _i32, _i32, _i64, _vp, _vp, _vp, _vp, _i32,
                                     _vp, _vp, _vp, _vp, _vp, _vp, _vp, _f32, _vp, _vp]
        lib.lrkv_prefill.restype = _i32
        lib.lrkv_prefill_chunk.argtypes = [_i32, _i32, _i32, _i32, _i32, _i64, _vp, _vp, _vp, _vp, _vp, _i32, _i32,
                                           _vp, _vp, _vp, _vp, _vp, _vp, _vp, _f32, _vp, _vp]
        lib.lrkv_prefill_chunk.restype = _i32
        lib.lrkv_pack_projection.argtypes = [_i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp]
        lib.lrkv_pack_projection.restype = _i32
        lib.lrkv_project_append.argtypes = [_i32, _i32, _i32, _i32, _i32, _i64, _vp, _vp, _vp, _vp, _vp, _i32, _i32,
                                            _vp, _vp, _vp, _sz, _vp]
        lib.lrkv_project_append.restype = _i32
        lib.lrkv_project_kernel.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32]
        lib.lrkv_project_workspace_size.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32, _i32, ctypes.POINTER(_sz)]
        lib.lrkv_project_workspace_size.restype = _i32
        lib.lrkv_project_kernel.restype = ctypes.c_char_p
        lib.lrkv_mha_decode_workspace_size.argtypes = [_i32, _i32, _i32, _i32, _i64, _i64, _i32, ctypes.POINTER(_sz)]
        lib.lrkv_mha_decode_workspace_size.restype = _i32
        lib.lrkv_mha_decode.argtypes = [_i32, _i32, _i32, _i32, _i64, _vp, _vp, _vp, _i64, _vp, _f32, _i32, _vp, _vp,
                                        _sz, _vp]
        lib.lrkv_mha_decode.restype = _i32
        lib.lrkv_train_forward.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                           _f32, _vp, _vp, _vp]
        lib.lrkv_train_forward.restype = _i32
        lib.lrkv_train_backward_workspace_size.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32, ctypes.POINTER(_sz)]
        lib.lrkv_train_backward_workspace_size.restype = _i32
        lib.lrkv_train_backward.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                            _vp, _vp, _vp, _f32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
        lib.lrkv_train_backward.restype = _i32
        _lib = lib
    return _lib


def lrkv_init() -> None:
    """Per-device set-up of the current device (kernel attributes, compute
    unit count); call before capturing library calls into a HIP graph."""
    _check(library().lrkv_init(), "lrkv_init")


def lrkv_status_string(status: int) -> str:
    return library().lrkv_status_string(int(status)).decode()


def lrkv_decode_scan_kernel(dtype: torch.dtype, num_heads: int, head_dim: int, rank: int) -> Optional[str]:
    """Name of the kernel lrkv_decode's scan runs on for these sizes (None if unsupported)."""
    name = library().lrkv_decode_scan_kernel(_dtype_code(dtype), num_heads, head_dim, rank)
    return None if name is None else name.decode()


def lrkv_cache_elems_per_token(num_heads: int, head_dim: int, rank: int) -> int:
    return int(library().lrkv_cache_elems_per_token(num_heads, head_dim, rank))


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return LRKV_BF16
    if t == torch.float32:
        return LRKV_F32
    raise LrkvError(3, f"unsupported dtype {t}")


def _ptr(t: Optional[torch.Tensor], name: str, dtype: Optional[torch.dtype] = None) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    return t.data_ptr() if t.numel() > 0 else None


def _shape(t: Optional[torch.Tensor], name: str, want: tuple) -> None:
    if t is not None and tuple(t.shape) != tuple(want):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(want)}")


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _check(status: int, where: str) -> None:
    if status != 0:
        raise LrkvError(status, where)


@dataclass
class LrkvCache:
    """Caller-owned cache tensors: shared rows [B, T, d_h] and latents [B, T, H, r]."""
    k_s: torch.Tensor
    v_s: torch.Tensor
    z_k: torch.Tensor
    z_v: torch.Tensor

    @property
    def batch(self) -> int: return self.k_s.shape[0]
    @property
    def capacity(self) -> int: return self.k_s.shape[1]
    @property
    def head_dim(self) -> int: return self.k_s.shape[2]
    @property
    def heads(self) -> int: return self.z_k.shape[2]
    @property
    def rank(self) -> int: return self.z_k.shape[3]
    @property
    def dtype(self) -> torch.dtype: return self.k_s.dtype

    @staticmethod
    def empty(batch, heads, head_dim, rank, capacity, dtype=torch.bfloat16, device="cuda", zero=True):
        mk = torch.zeros if zero else torch.empty
        return LrkvCache(mk((batch, capacity, head_dim), dtype=dtype, device=device),
                         mk((batch, capacity, head_dim), dtype=dtype, device=device),
                         mk((batch, capacity, heads, rank), dtype=dtype, device=device),
                         mk((batch, capacity, heads, rank), dtype=dtype, device=device))

    def check(self):
        B, T, d_h = self.k_s.shape
        H, r = self.z_k.shape[2], self.z_k.shape[3]
        _shape(self.v_s, "v_s", (B, T, d_h))
        _shape(self.z_k, "z_k", (B, T, H, r))
        _shape(self.z_v, "z_v", (B, T, H, r))
        for t, n in ((self.v_s, "v_s"), (self.z_k, "z_k"), (self.z_v, "z_v")):
            if t.dtype != self.dtype or t.device != self.k_s.device:
                raise ValueError(f"cache tensor {n} differs in dtype/device from k_s")

    def pointers(self):
        self.check()
        dt = self.dtype
        return (_ptr(self.k_s, "k_s", dt), _ptr(self.v_s, "v_s", dt), _ptr(self.z_k, "z_k", dt),
                _ptr(self.z_v, "z_v", dt))


def lrkv_append(cache: LrkvCache, pos: torch.Tensor, new_k_s, new_v_s, new_z_k, new_z_v) -> None:
    dt = cache.dtype
    B, n_new = new_k_s.shape[0], new_k_s.shape[1]
    if B != cache.batch:
        raise ValueError("new rows and cache differ in batch")
    _shape(new_k_s, "new_k_s", (B, n_new, cache.head_dim))
    _shape(new_v_s, "new_v_s", (B, n_new, cache.head_dim))
    _shape(new_z_k, "new_z_k", (B, n_new, cache.heads, cache.rank))
    _shape(new_z_v, "new_z_v", (B, n_new, cache.heads, cache.rank))
    _shape(pos, "pos", (B,))
    _check(library().lrkv_append(_dtype_code(dt), cache.batch, cache.heads, cache.head_dim, cache.rank,
                                 cache.capacity, *cache.pointers(), _ptr(pos, "pos", torch.int32), n_new,
                                 _ptr(new_k_s, "new_k_s", dt), _ptr(new_v_s, "new_v_s", dt),
                                 _ptr(new_z_k, "new_z_k", dt), _ptr(new_z_v, "new_z_v", dt), _stream()),
           "lrkv_append")


def lrkv_decode_workspace_size(dtype: torch.dtype, batch: int, heads: int, head_dim: int, rank: int,
                               capacity: int, max_len: int, split_tokens: int = 0) -> int:
    n = _sz(0)
    _check(library().lrkv_decode_workspace_size(_dtype_code(dtype), batch, heads, head_dim, rank, capacity,
                                                max_len, split_tokens, ctypes.byref(n)),
           "lrkv_decode_workspace_size")
    return int(n.value)


def lrkv_decode_workspace_size_ex(engine: int, dtype: torch.dtype, batch: int, heads: int, head_dim: int, rank: int,
                                  capacity: int, max_len: int, split_tokens: int = 0) -> int:
    n = _sz(0)
    _check(library().lrkv_decode_workspace_size_ex(int(engine), _dtype_code(dtype), batch, heads, head_dim, rank,
                                                   capacity, max_len, split_tokens, ctypes.byref(n)),
           "lrkv_decode_workspace_size_ex")
    return int(n.value)


def decode_workspace(cache: LrkvCache, max_len: int, split_tokens: int = 0, engine: int = 0) -> torch.Tensor:
    nbytes = lrkv_decode_workspace_size_ex(engine, cache.dtype, cache.batch, cache.heads, cache.head_dim,
                                           cache.rank, cache.capacity, max_len, split_tokens)
    return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=cache.k_s.device)


def lrkv_decode(cache: LrkvCache, seq_lens: torch.Tensor, max_len: int, q: torch.Tensor, b_k: torch.Tensor,
                b_v: torch.Tensor, scale: Optional[float] = None, split_tokens: int = 0,
                out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                phase: str = "both", engine: int = 0) -> torch.Tensor:
    """phase: "both" (lrkv_decode), "partial" (lrkv_decode_partial) or "combine" (lrkv_decode_combine);
    engine != 0 goes through lrkv_decode_ex (1: vector-ALU scan, 2: MFMA scan, 3: any-rank scan,
    4: any-rank MFMA scan)."""
    dt = cache.dtype
    B, H, d_h, r = cache.batch, cache.heads, cache.head_dim, cache.rank
    _shape(q, "q", (B, H, d_h))
    _shape(b_k, "b_k", (H, d_h, r))
    _shape(b_v, "b_v", (H, d_h, r))
    _shape(seq_lens, "seq_lens", (B,))
    if out is None:
        out = torch.empty_like(q)
    _shape(out, "out", (B, H, d_h))
    if workspace is None:
        workspace = decode_workspace(cache, max_len, split_tokens, engine)
    if engine:
        phases = {"both": 3, "partial": 1, "combine": 2}[phase]
        fn = lambda *a: library().lrkv_decode_ex(int(engine), phases, *a)
    else:
        fn = {"both": library().lrkv_decode, "partial": library().lrkv_decode_partial,
              "combine": library().lrkv_decode_combine}[phase]
    _check(fn(_dtype_code(dt), cache.batch, cache.heads, cache.head_dim, cache.rank,
                                 cache.capacity, *cache.pointers(), _ptr(seq_lens, "seq_lens", torch.int32),
                                 max_len, _ptr(q, "q", dt), _ptr(b_k, "b_k", dt), _ptr(b_v, "b_v", dt),
                                 0.0 if scale is None else float(scale), split_tokens, _ptr(out, "out", dt),
                                 _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
                                 _stream()),
           "lrkv_decode")
    return out


def lrkv_decode_noalloc(cache: LrkvCache, seq_lens: torch.Tensor, max_len: int, q: torch.Tensor, b_k: torch.Tensor,
                        b_v: torch.Tensor, scale: Optional[float] = None, split_tokens: int = 0,
                        out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """lrkv_decode without a workspace: the partial states go to the library's
    fixed per-device scratch (see lrkv.h).  Pass `out` to allocate nothing."""
    dt = cache.dtype
    B, H, d_h, r = cache.batch, cache.heads, cache.head_dim, cache.rank
    _shape(q, "q", (B, H, d_h))
    _shape(b_k, "b_k", (H, d_h, r))
    _shape(b_v, "b_v", (H, d_h, r))
    _shape(seq_lens, "seq_lens", (B,))
    if out is None:
        out = torch.empty_like(q)
    _shape(out, "out", (B, H, d_h))
    _check(library().lrkv_decode_noalloc(_dtype_code(dt), B, H, d_h, r, cache.capacity, *cache.pointers(),
                                         _ptr(seq_lens, "seq_lens", torch.int32), max_len, _ptr(q, "q", dt),
                                         _ptr(b_k, "b_k", dt), _ptr(b_v, "b_v", dt),
                                         0.0 if scale is None else float(scale), split_tokens,
                                         _ptr(out, "out", dt), _stream()),
           "lrkv_decode_noalloc")
    return out


class DecodeCall:
    """A decode whose arguments are marshalled once: the three methods call
    lrkv_decode, lrkv_decode_partial and lrkv_decode_combine with the same
    tensors on torch's current stream at the time of each call.  The tensors
    must stay alive and keep their shapes; this only removes the per-call
    argument checking from loops that repeat the same decode."""

    def __init__(self, cache: LrkvCache, seq_lens, max_len, q, b_k, b_v, scale=None, split_tokens=0,
                 out=None, workspace=None, engine=0):
        self.out = out if out is not None else torch.empty_like(q)
        self.workspace = (workspace if workspace is not None
                          else decode_workspace(cache, max_len, split_tokens, engine))
        # validate once through the regular path (a real call), then freeze the argument tuple
        lrkv_decode(cache, seq_lens, max_len, q, b_k, b_v, scale, split_tokens, self.out, self.workspace,
                    phase="partial", engine=engine)
        dt = cache.dtype
        self._keep = (cache, seq_lens, q, b_k, b_v)
        self._args = (_dtype_code(dt), cache.batch, cache.heads, cache.head_dim, cache.rank, cache.capacity,
                      *cache.pointers(), _ptr(seq_lens, "seq_lens", torch.int32), max_len, _ptr(q, "q", dt),
                      _ptr(b_k, "b_k", dt), _ptr(b_v, "b_v", dt), 0.0 if scale is None else float(scale),
                      split_tokens, _ptr(self.out, "out", dt), _ptr(self.workspace, "workspace"),
                      self.workspace.numel())
        lib = library()
        if engine:
            ex = lib.lrkv_decode_ex
            self._fns = tuple((lambda ph: (lambda *a: ex(int(engine), ph, *a)))(ph) for ph in (3, 1, 2))
        else:
            self._fns = (lib.lrkv_decode, lib.lrkv_decode_partial, lib.lrkv_decode_combine)

    def _call(self, i):
        st = self._fns[i](*self._args, torch.cuda.current_stream().cuda_stream)
        if st != 0:
            raise LrkvError(st, ("lrkv_decode", "lrkv_decode_partial", "lrkv_decode_combine")[i])

    def both(self):
        self._call(0)

    def partial(self):
        self._call(1)

    def combine(self):
        self._call(2)


def lrkv_prefill_kernel(dtype: torch.dtype, num_heads: int, head_dim: int, rank: int) -> Optional[str]:
    """Name of the kernel lrkv_prefill runs on for these sizes (None if unsupported)."""
    name = library().lrkv_prefill_kernel(_dtype_code(dtype), num_heads, head_dim, rank)
    return None if name is None else name.decode()


def lrkv_prefill(q, k_s, v_s, z_k, z_v, b_k, b_v, scale: Optional[float] = None,
                 cache: Optional[LrkvCache] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    dt = q.dtype
    B, L, H, d_h = q.shape
    r = z_k.shape[-1]
    _shape(k_s, "k_s", (B, L, d_h))
    _shape(v_s, "v_s", (B, L, d_h))
    _shape(z_k, "z_k", (B, L, H, r))
    _shape(z_v, "z_v", (B, L, H, r))
    _shape(b_k, "b_k", (H, d_h, r))
    _shape(b_v, "b_v", (H, d_h, r))
    if out is None:
        out = torch.empty_like(q)
    _shape(out, "out", (B, L, H, d_h))
    if cache is not None and (cache.batch, cache.heads, cache.head_dim, cache.rank) != (B, H, d_h, r):
        raise ValueError("cache dimensions differ from the prefill inputs")
    cptr = cache.pointers() if cache is not None else (None, None, None, None)
    cap = cache.capacity if cache is not None else max(L, 1)
    _check(library().lrkv_prefill(_dtype_code(dt), B, H, d_h, r, cap, *cptr, L, _ptr(q, "q", dt),
                                  _ptr(k_s, "k_s", dt), _ptr(v_s, "v_s", dt), _ptr(z_k, "z_k", dt),
                                  _ptr(z_v, "z_v", dt), _ptr(b_k, "b_k", dt), _ptr(b_v, "b_v", dt),
                                  0.0 if scale is None else float(scale), _ptr(out, "out", dt), _stream()),
           "lrkv_prefill")
    return out


def lrkv_prefill_chunk(cache: LrkvCache, start_pos: torch.Tensor, max_start: int, q, k_s, v_s, z_k, z_v, b_k, b_v,
                       scale: Optional[float] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """New tokens over cached history: writes them at slots start_pos[b].. of the
    cache and returns their causal attention over the cache (see lrkv.h)."""
    dt = q.dtype
    B, L, H, d_h = q.shape
    r = z_k.shape[-1]
    _shape(k_s, "k_s", (B, L, d_h))
    _shape(v_s, "v_s", (B, L, d_h))
    _shape(z_k, "z_k", (B, L, H, r))
    _shape(z_v, "z_v", (B, L, H, r))
    _shape(b_k, "b_k", (H, d_h, r))
    _shape(b_v, "b_v", (H, d_h, r))
    if (cache.batch, cache.heads, cache.head_dim, cache.rank) != (B, H, d_h, r):
        raise ValueError("cache dimensions differ from the chunk inputs")
    _shape(start_pos, "start_pos", (B,))
    if out is None:
        out = torch.empty_like(q)
    _shape(out, "out", (B, L, H, d_h))
    _check(library().lrkv_prefill_chunk(_dtype_code(dt), B, H, d_h, r, cache.capacity, *cache.pointers(),
                                        _ptr(start_pos, "start_pos", torch.int32), int(max_start), L,
                                        _ptr(q, "q", dt),
                                        _ptr(k_s, "k_s", dt), _ptr(v_s, "v_s", dt), _ptr(z_k, "z_k", dt),
                                        _ptr(z_v, "z_v", dt), _ptr(b_k, "b_k", dt), _ptr(b_v, "b_v", dt),
                                        0.0 if scale is None else float(scale), _ptr(out, "out", dt), _stream()),
           "lrkv_prefill_chunk")
    return out


def lrkv_pack_projection(wk_shared, wv_shared, u_k, u_v, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Packed projection weight [2(d_h + H r)][d] from W^K_shared, W^V_shared
    [d][d_h] and U^K, U^V [H][d][r] (see lrkv.h)."""
    dt = wk_shared.dtype
    d, d_h = wk_shared.shape
    H, _, r = u_k.shape
    _shape(wv_shared, "wv_shared", (d, d_h))
    _shape(u_k, "u_k", (H, d, r))
    _shape(u_v, "u_v", (H, d, r))
    if out is None:
        out = torch.empty(2 * (d_h + H * r), d, dtype=dt, device=wk_shared.device)
    _shape(out, "out", (2 * (d_h + H * r), d))
    _check(library().lrkv_pack_projection(_dtype_code(dt), H, d_h, r, d, _ptr(wk_shared, "wk_shared", dt),
                                          _ptr(wv_shared, "wv_shared", dt), _ptr(u_k, "u_k", dt),
                                          _ptr(u_v, "u_v", dt), _ptr(out, "out", dt), _stream()),
           "lrkv_pack_projection")
    return out


def lrkv_project_kernel(dtype: torch.dtype, batch: int, n_new: int, heads: int, head_dim: int, rank: int,
                        d_model: int, with_workspace: bool = True) -> Optional[str]:
    """Name of the kernel lrkv_project_append runs for these sizes (None if invalid)."""
    name = library().lrkv_project_kernel(_dtype_code(dtype), batch, n_new, heads, head_dim, rank, d_model,
                                         int(bool(with_workspace)))
    return None if name is None else name.decode()


def lrkv_project_workspace_size(dtype: torch.dtype, batch: int, n_new: int, heads: int, head_dim: int, rank: int,
                                d_model: int) -> int:
    n = _sz(0)
    _check(library().lrkv_project_workspace_size(_dtype_code(dtype), batch, n_new, heads, head_dim, rank, d_model,
                                                 ctypes.byref(n)),
           "lrkv_project_workspace_size")
    return int(n.value)


def lrkv_project_append(cache: LrkvCache, pos: torch.Tensor, x: torch.Tensor, w_packed: torch.Tensor,
                        workspace="auto") -> None:
    """Fused projection + append: the cache rows of x [B][n_new][d] computed
    with the packed weight and written at slots pos[b].. (see lrkv.h).
    workspace: "auto" allocates the one the sizes can use, None passes none,
    or a uint8 device tensor."""
    dt = cache.dtype
    B, n_new, d = x.shape
    if B != cache.batch:
        raise ValueError("x and cache differ in batch")
    _shape(w_packed, "w_packed", (2 * (cache.head_dim + cache.heads * cache.rank), d))
    _shape(pos, "pos", (B,))
    if isinstance(workspace, str):
        nbytes = lrkv_project_workspace_size(dt, B, n_new, cache.heads, cache.head_dim, cache.rank, d) if n_new else 0
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=x.device) if nbytes else None
    ws_ptr = _ptr(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() if workspace is not None else 0
    _check(library().lrkv_project_append(_dtype_code(dt), cache.batch, cache.heads, cache.head_dim, cache.rank,
                                         cache.capacity, *cache.pointers(), _ptr(pos, "pos", torch.int32), n_new,
                                         d, _ptr(x, "x", dt), _ptr(w_packed, "w_packed", dt), ws_ptr, ws_bytes,
                                         _stream()),
           "lrkv_project_append")


def lrkv_mha_decode_workspace_size(dtype: torch.dtype, batch: int, heads: int, head_dim: int, capacity: int,
                                   max_len: int, split_tokens: int = 0) -> int:
    n = _sz(0)
    _check(library().lrkv_mha_decode_workspace_size(_dtype_code(dtype), batch, heads, head_dim, capacity, max_len,
                                                    split_tokens, ctypes.byref(n)),
           "lrkv_mha_decode_workspace_size")
    return int(n.value)


def lrkv_mha_decode(k: torch.Tensor, v: torch.Tensor, seq_lens: torch.Tensor, max_len: int, q: torch.Tensor,
                    scale: Optional[float] = None, split_tokens: int = 0, out: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Plain MHA decode over a per-head cache k, v [B][T][H][d_h] (see lrkv.h)."""
    dt = q.dtype
    B, T, H, d_h = k.shape
    _shape(v, "v", (B, T, H, d_h))
    _shape(q, "q", (B, H, d_h))
    _shape(seq_lens, "seq_lens", (B,))
    if out is None:
        out = torch.empty_like(q)
    _shape(out, "out", (B, H, d_h))
    if workspace is None:
        nbytes = lrkv_mha_decode_workspace_size(dt, B, H, d_h, T, max_len, split_tokens)
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    _check(library().lrkv_mha_decode(_dtype_code(dt), B, H, d_h, T, _ptr(k, "k", dt), _ptr(v, "v", dt),
                                     _ptr(seq_lens, "seq_lens", torch.int32), int(max_len), _ptr(q, "q", dt),
                                     0.0 if scale is None else float(scale), split_tokens, _ptr(out, "out", dt),
                                     _ptr(workspace, "workspace"), workspace.numel(), _stream()),
           "lrkv_mha_decode")
    return out


def _train_shapes(q, k_s, v_s, z_k, z_v, b_k, b_v):
    B, L, H, d_h = q.shape
    r = z_k.shape[-1]
    _shape(k_s, "k_s", (B, L, d_h))
    _shape(v_s, "v_s", (B, L, d_h))
    _shape(z_k, "z_k", (B, L, H, r))
    _shape(z_v, "z_v", (B, L, H, r))
    _shape(b_k, "b_k", (H, d_h, r))
    _shape(b_v, "b_v", (H, d_h, r))
    return B, L, H, d_h, r


def lrkv_train_forward(q, k_s, v_s, z_k, z_v, b_k, b_v, scale: Optional[float] = None,
                       out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None):
    """Causal LRKV attention over fresh sequences, returning (out, lse) with
    lse[b, i, h] the natural log-sum-exp of row i's scaled logits (fp32)."""
    dt = q.dtype
    B, L, H, d_h, r = _train_shapes(q, k_s, v_s, z_k, z_v, b_k, b_v)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(B, L, H, dtype=torch.float32, device=q.device)
    _shape(out, "out", (B, L, H, d_h))
    _shape(lse, "lse", (B, L, H))
    _check(library().lrkv_train_forward(_dtype_code(dt), B, H, d_h, r, L, _ptr(q, "q", dt), _ptr(k_s, "k_s", dt),
                                        _ptr(v_s, "v_s", dt), _ptr(z_k, "z_k", dt), _ptr(z_v, "z_v", dt),
                                        _ptr(b_k, "b_k", dt), _ptr(b_v, "b_v", dt),
                                        0.0 if scale is None else float(scale), _ptr(out, "out", dt),
                                        _ptr(lse, "lse", torch.float32), _stream()),
           "lrkv_train_forward")
    return out, lse


def lrkv_train_backward_workspace_size(dtype: torch.dtype, batch: int, heads: int, head_dim: int, rank: int,
                                       seq_len: int) -> int:
    n = _sz(0)
    _check(library().lrkv_train_backward_workspace_size(_dtype_code(dtype), batch, heads, head_dim, rank, seq_len,
                                                        ctypes.byref(n)), "lrkv_train_backward_workspace_size")
    return n.value


def lrkv_train_backward(q, k_s, v_s, z_k, z_v, b_k, b_v, out, lse, d_out, scale: Optional[float] = None,
                        workspace: Optional[torch.Tensor] = None, grads: Optional[dict] = None) -> dict:
    """Gradients (fp32) of the loss with upstream gradient d_out through
    lrkv_train_forward: dict with dq, dk_s, dv_s, dz_k, dz_v, db_k, db_v."""
    dt = q.dtype
    B, L, H, d_h, r = _train_shapes(q, k_s, v_s, z_k, z_v, b_k, b_v)
    _shape(out, "out", (B, L, H, d_h))
    _shape(lse, "lse", (B, L, H))
    _shape(d_out, "d_out", (B, L, H, d_h))
    dev, f32 = q.device, torch.float32
    if grads is None:
        grads = {"dq": torch.empty(B, L, H, d_h, dtype=f32, device=dev),
                 "dk_s": torch.empty(B, L, d_h, dtype=f32, device=dev),
                 "dv_s": torch.empty(B, L, d_h, dtype=f32, device=dev),
                 "dz_k": torch.empty(B, L, H, r, dtype=f32, device=dev),
                 "dz_v": torch.empty(B, L, H, r, dtype=f32, device=dev),
                 "db_k": torch.empty(H, d_h, r, dtype=f32, device=dev),
                 "db_v": torch.empty(H, d_h, r, dtype=f32, device=dev)}
    need = lrkv_train_backward_workspace_size(dt, B, H, d_h, r, L)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    g = {k: _ptr(v, k, f32) for k, v in grads.items()}
    _check(library().lrkv_train_backward(
        _dtype_code(dt), B, H, d_h, r, L, _ptr(q, "q", dt), _ptr(k_s, "k_s", dt), _ptr(v_s, "v_s", dt),
        _ptr(z_k, "z_k", dt), _ptr(z_v, "z_v", dt), _ptr(b_k, "b_k", dt), _ptr(b_v, "b_v", dt),
        _ptr(out, "out", dt), _ptr(lse, "lse", f32), _ptr(d_out, "d_out", dt),
        0.0 if scale is None else float(scale), g["dq"], g["dk_s"], g["dv_s"], g["dz_k"], g["dz_v"], g["db_k"],
        g["db_v"], _ptr(workspace, "workspace"), workspace.numel(), _stream()), "lrkv_train_backward")
    return grads


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)
