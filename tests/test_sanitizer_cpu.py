"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU needed).

Every source of libgqa is compiled with the sanitizers on its host side only (device code is
built as usual), linked into a separate library, and the host-side ABI tests
(tests/test_abi_cpu.py: argument validation, every error path, workspace queries, symbol
exports) run against that build in a child process with the sanitizer runtime preloaded.  Any
out-of-bounds access, use after free or undefined behaviour in the validation and sizing code
aborts the child, and the test fails.
"""

import glob
import os
import subprocess
import sys

import pytest

from gqa_causal_flash_amd import build as gbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
# host-side only: each sanitizer flag reaches the host compilation, never the gfx950 one
HOST_SANITIZE = [
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined",
    "-Xarch_host", "-fno-omit-frame-pointer",
    "-g",
]


def _runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


@pytest.mark.skipif(_runtime() is None, reason="clang's ASan runtime is not installed")
def test_abi_host_code_is_clean_under_asan_and_ubsan(tmp_path):
    lib = str(tmp_path / "libgqa_sanitized.so")
    # the sanitizer runtime is preloaded into the child, so the library resolves its hooks there
    gbuild.build(extra_flags=HOST_SANITIZE, out=lib)
    env = dict(os.environ)
    env.update(
        LD_PRELOAD=_runtime(),
        GQA_LIBRARY=lib,
        ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
        UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1",
    )
    probe = ("import ctypes, gqa_causal_flash_amd as g; "
             "assert g.lib_path() == %r; ctypes.CDLL(None).__asan_init; print('sanitized build loaded')" % lib)
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and "sanitized build loaded" in r.stdout, r.stdout + r.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "tests/test_abi_cpu.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    print(r.stdout[-2000:], r.stderr[-4000:])
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
    assert " passed" in r.stdout
