"""The C ABI's host side under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The library is rebuilt with the sanitizers on its host code only (every -fsanitize= follows
-Xarch_host; the gfx950 device code is compiled as usual), and tests/test_abi_cpu.py -- the
argument validation, workspace sizing, launch-count query and status strings, called with
fake device pointers so that nothing is launched -- runs against it in a child process with the
sanitizer runtime preloaded.  Any out-of-bounds access, use of uninitialised or freed memory,
signed overflow or other undefined behaviour in that code fails the test.
"""

import glob
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


@pytest.mark.skipif(_asan_runtime() is None, reason="no clang AddressSanitizer runtime in this ROCm")
def test_abi_checks_under_sanitizers():
    from compressed_sparse_long_c4a_amd import build
    with tempfile.TemporaryDirectory(prefix="csa_san_") as tmp:
        lib = os.path.join(tmp, "libcsa_san.so")
        build.build(out=lib, extra_flags=SAN, link_flags=["-Xarch_host", "-shared-libasan", *SAN])
        code = (f"import sys; sys.path.insert(0, {ROOT!r}); "
                "import compressed_sparse_long_c4a_amd as csa; "
                f"csa.LIB_PATH = {lib!r}; import pytest; "
                f"sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', {os.path.join(ROOT, 'tests', 'test_abi_cpu.py')!r}]))")
        env = dict(os.environ, LD_PRELOAD=_asan_runtime(),
                   ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
                   UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
        r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=600)
        print(r.stdout[-3000:], r.stderr[-3000:])
        assert r.returncode == 0, "sanitized ABI checks failed"
        assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr
        assert "runtime error" not in r.stderr
