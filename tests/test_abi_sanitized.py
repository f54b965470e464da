"""The C-ABI host tests (tests/test_abi.py) rerun against the host-sanitizer
build of the library (AddressSanitizer + UndefinedBehaviorSanitizer on the
host code of lrkv_api.hip: validation, planning, workspace layout), in a
child process with the sanitizer runtime preloaded.  Any sanitizer report
aborts the child (halt_on_error), so a green run means none fired.
CPU only: every case fails host validation before any launch."""
import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(torch.cuda.is_available(), reason="host-validation cases use fake device pointers")
def test_abi_under_asan_and_ubsan():
    from rank_compressed_kv_lrkv_amd import build_sanitized as bs
    if not os.path.exists(bs.SAN_LIB):
        pytest.skip("the sanitizer build is made by __graft_entry__.build()")
    env = dict(os.environ)
    env.update(LD_PRELOAD=bs.runtime(), ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", LRKV_LIBRARY=bs.SAN_LIB,
               PYTHONPATH=ROOT + os.pathsep + env.get("PYTHONPATH", ""))
    probe = ("import rank_compressed_kv_lrkv_amd.binding as B, ctypes; B.library(); "
             "print(B.LIB_PATH); print(hasattr(ctypes.CDLL(B.LIB_PATH), '__asan_init'))")
    res = subprocess.run([sys.executable, "-c", probe], env=env, cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stderr[-4000:]
    assert res.stdout.split() == [bs.SAN_LIB, "True"], res.stdout
    res = subprocess.run([sys.executable, "-m", "pytest", "tests/test_abi.py", "-q", "-m", "not gpu",
                          "-p", "no:cacheprovider"], env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    print(res.stdout[-3000:])
    assert res.returncode == 0, res.stdout[-3000:] + res.stderr[-3000:]
