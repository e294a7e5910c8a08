"""Host sanitizer runs (CPU only): the oracle built with AddressSanitizer and UndefinedBehaviorSanitizer runs every
oracle pin, and the C ABI's host code built the same way runs every host-side ABI test.  Each run happens in a
child process with the sanitizer runtime preloaded and stops at the first report; a planted out-of-bounds write
shows that the instrumented oracle does report.  GPU code is never instrumented: the ABI's device code is compiled
as usual, and the sanitizer flags apply to its host pass only."""
import glob
import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402

SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}
GCC_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]


def _gcc_runtime():
    p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def _run(code, preload, timeout=600):
    env = dict(os.environ, LD_PRELOAD=preload, PYTHONPATH=ROOT, **SAN_ENV)
    return subprocess.run([sys.executable, "-c", textwrap.dedent(code)], cwd=ROOT, env=env, capture_output=True,
                          text=True, timeout=timeout)


@pytest.fixture(scope="module")
def asan_oracle(tmp_path_factory):
    rt = _gcc_runtime()
    if rt is None:
        pytest.skip("gcc has no AddressSanitizer runtime here")
    out = str(tmp_path_factory.mktemp("asan") / "liboracle_asan.so")
    oracle.build(out=out, extra_flags=GCC_FLAGS)
    return out, rt


def test_oracle_pins_under_asan_ubsan(asan_oracle):
    lib, rt = asan_oracle
    r = _run("""
        import sys
        import oracle
        oracle._default = oracle.Oracle(%r)
        import pytest
        sys.exit(pytest.main(["-q", "-x", "-s", "-p", "no:cacheprovider", "tests/test_oracle_pins.py"]))
    """ % lib, rt)
    assert r.returncode == 0 and "passed" in r.stdout, r.stdout[-3000:] + r.stderr[-3000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-3000:]


def test_planted_overflow_is_reported(asan_oracle, tmp_path):
    """The same build of a copy of the oracle with one planted out-of-bounds write stops with a report."""
    _, rt = asan_oracle
    src = tmp_path / "planted.c"
    src.write_text(open(os.path.join(ROOT, "oracle", "efla_oracle.c")).read() + textwrap.dedent("""
        #include <stdlib.h>
        double planted_overflow(int n) {
            double* a = (double*)malloc(sizeof(double) * (size_t)n);
            for (int i = 0; i <= n; ++i) a[i] = i;   /* one past the end */
            const double s = a[0];
            free(a);
            return s;
        }
    """))
    lib = str(tmp_path / "libplanted.so")
    oracle.build(src=str(src), out=lib, extra_flags=GCC_FLAGS)
    r = _run("""
        import ctypes
        ctypes.CDLL(%r).planted_overflow(8)
    """ % lib, rt)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, r.stderr[-3000:]


@pytest.fixture(scope="module")
def asan_abi(tmp_path_factory):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    rts = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    objs = [o for o in sorted(glob.glob(os.path.join(ROOT, "_build", "*.o"))) if not o.endswith("efla_api.o")]
    if not os.path.exists(hipcc) or not rts or not objs:
        pytest.skip("needs hipcc, its AddressSanitizer runtime and the built objects of the library")
    d = tmp_path_factory.mktemp("asan_abi")
    api_o, lib = str(d / "efla_api_san.o"), str(d / "libefla_san.so")
    # the sanitizers instrument the host pass only (each flag behind -Xarch_host); the device code is unchanged
    cmd = [hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "exact_flow_delta_amd", "csrc"),
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer",
           "-c", os.path.join(ROOT, "exact_flow_delta_amd", "csrc", "efla_api.hip"), "-o", api_o]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    # linked without the runtime: its symbols come from the preloaded one
    r = subprocess.run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", lib, api_o] + objs,
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return lib, rts[-1]


def test_abi_host_checks_under_asan_ubsan(asan_abi):
    lib, rt = asan_abi
    r = _run("""
        import sys
        import exact_flow_delta_amd as efla
        efla._LIB_PATH = %r
        efla.load_library()
        import pytest
        sys.exit(pytest.main(["-q", "-x", "-s", "-p", "no:cacheprovider", "tests/test_abi_cpu.py"]))
    """ % lib, rt)
    assert r.returncode == 0 and "passed" in r.stdout, r.stdout[-3000:] + r.stderr[-3000:]
    assert "runtime error" not in r.stdout + r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-3000:]
