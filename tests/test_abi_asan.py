"""The C ABI's host-side argument validation under AddressSanitizer (CPU only, no GPU needed).

The library is rebuilt with its host code instrumented (device code unchanged) into a temporary directory, and
tests/test_abi.py runs against that build in a child process with the sanitizer's runtime preloaded: every
validation path those tests reach (null pointers, bad sizes, dtypes, chunk lengths, position and length ranges,
workspace sizes and their queries) then runs with out-of-bounds, use-after-free and similar checks on.
"""
import concurrent.futures as cf
import glob
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "root_parity_gated_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def _build(out_dir):
    flags = ["-std=c++17", "-O1", "-g", "-fPIC", "--offload-arch=gfx950",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
             f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]

    def one(src):
        obj = os.path.join(out_dir, os.path.basename(src).replace(".hip", ".o"))
        r = subprocess.run([HIPCC, *flags, "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        return obj

    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(one, srcs))
    lib = os.path.join(out_dir, "libsanatan_asan.so")
    r = subprocess.run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address",
                        "-shared-libasan", "-o", lib, *objs], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return lib


def test_abi_validation_under_asan(tmp_path):
    import pytest

    rt = _asan_runtime()
    if rt is None or not os.path.exists(HIPCC):
        pytest.skip("no hipcc or clang ASan runtime")
    lib = _build(str(tmp_path))
    # the host code really is instrumented: it calls the sanitizer's checks
    nm = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report_load" in nm or "__asan_report_store" in nm
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               SANATAN_TEST_LIB=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q", "-x",
                        "-p", "no:cacheprovider"], cwd=str(tmp_path), env=env, capture_output=True, text=True,
                       timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
