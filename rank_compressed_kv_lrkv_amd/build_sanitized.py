"""Host-sanitizer build of the C-ABI layer: lib/liblrkv_san.so.

The host code of csrc/lrkv_api.hip (argument validation, planning,
workspace layout, status codes) is compiled with AddressSanitizer and
UndefinedBehaviorSanitizer; the kernels' objects are the ones the ordinary
build made (`build.py`), so the device code is the same.  Load it with the
sanitizer runtime preloaded and LRKV_LIBRARY naming it, e.g.

    LD_PRELOAD=$(python -m rank_compressed_kv_lrkv_amd.build_sanitized --runtime) \\
    ASAN_OPTIONS=detect_leaks=0 LRKV_LIBRARY=.../lib/liblrkv_san.so python -m pytest tests/test_abi.py

(tests/test_abi_sanitized.py runs exactly that).  Device code is never built
with a sanitizer: the flags apply to the host compilation only.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

from .build import ARCH, HIPCC_FLAGS, LIB_DIR, OBJ, SRC, hipcc

SAN_LIB = os.path.join(LIB_DIR, "liblrkv_san.so")
HOST_SANITIZE = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -Xarch_host -fno-omit-frame-pointer"


def runtime() -> str:
    """Path of the shared ASan runtime (with the UBSan handlers) of the ROCm clang."""
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("ASan runtime not found under /opt/rocm/llvm")
    return hits[-1]


def build_sanitized(verbose: bool = True) -> str:
    api = os.path.join(SRC, "lrkv_api.hip")
    san_obj = os.path.join(OBJ, "lrkv_api.san.o")
    flags = [f for f in HIPCC_FLAGS if f not in ("-O3",)] + ["-O1", "-g", *HOST_SANITIZE.split()]
    res = subprocess.run([hipcc(), *flags, "-c", api, "-o", san_obj], capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"sanitized compile failed:\n{res.stderr[-8000:]}")
    others = [os.path.join(OBJ, os.path.basename(s) + ".o") for s in sorted(glob.glob(os.path.join(SRC, "*.hip")))
              if os.path.basename(s) != "lrkv_api.hip"]
    missing = [o for o in others if not os.path.exists(o)]
    if missing:
        raise RuntimeError(f"run the ordinary build first; missing {missing}")
    tmp = SAN_LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *HOST_SANITIZE.split(), "-shared-libsan",
           san_obj, *others, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"sanitized link failed:\n{res.stderr[-8000:]}")
    os.replace(tmp, SAN_LIB)
    if verbose:
        print(f"built {SAN_LIB} (host code of lrkv_api.hip with ASan + UBSan)", file=sys.stderr)
    return SAN_LIB


if __name__ == "__main__":
    if "--runtime" in sys.argv:
        print(runtime())
    else:
        build_sanitized()
