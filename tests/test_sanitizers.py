"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The oracle (oracle.c) and the C-ABI unit of the library (api.hip, host pass) are rebuilt with
clang's ASan + UBSan, and the whole CPU suite (oracle pins and ABI checks) runs against those
builds in a child process that preloads the ASan runtime.  A planted heap overflow in a
throw-away C file, built and loaded the same way, must be reported: that shows the harness
really runs instrumented code."""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from routed_expert_ffn_route_amd import build as libbuild  # noqa: E402

pytestmark = pytest.mark.skipif(not os.path.exists(oracle.CLANG), reason="clang (ROCm LLVM) is not installed")


def _env(extra):
    env = dict(os.environ)
    env.update({"LD_PRELOAD": oracle.asan_runtime(), "ASAN_OPTIONS": "detect_leaks=0",
                "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"})
    env.update(extra)
    return env


@pytest.fixture(scope="module")
def san_dir():
    with tempfile.TemporaryDirectory() as d:
        yield d


def test_harness_reports_a_planted_overflow(san_dir):
    src = os.path.join(san_dir, "planted.c")
    with open(src, "w") as f:
        f.write("#include <stdlib.h>\nint planted(int i) { int *p = malloc(4 * sizeof(int)); "
                "int v = p[i]; free(p); return v; }\n")
    so = os.path.join(san_dir, "libplanted.so")
    subprocess.run([oracle.CLANG, "-O1", "-g", "-fsanitize=address", "-shared-libsan", "-fPIC", "-shared",
                    "-o", so, src], check=True)
    code = f"import ctypes; ctypes.CDLL({so!r}).planted(4)"
    r = subprocess.run([sys.executable, "-c", code], env=_env({}), capture_output=True, text=True, timeout=120)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr


def test_cpu_suite_clean_under_asan_ubsan(san_dir):
    orc = oracle.build_sanitized(san_dir)
    try:
        moe = libbuild.build_sanitized(san_dir)
    except RuntimeError as e:  # no objects of a previous build to link against
        pytest.skip(str(e))
    env = _env({"MOE_ORACLE_LIB": orc, "MOE_LIB": moe})
    # the child loads both instrumented builds (checked through its memory map) ...
    probe = ("import oracle; from routed_expert_ffn_route_amd import binding as B; oracle.lib(); B.lib(); "
             "m = open('/proc/self/maps').read(); print('liboracle_san.so' in m, 'libmoe_san.so' in m)")
    r = subprocess.run([sys.executable, "-c", probe], env=env, cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.split() == ["True", "True"], r.stderr[-2000:]
    # ... and runs the oracle pins and the ABI checks with every report fatal
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_oracle_pins.py", "tests/test_abi.py", "-q",
                        "-m", "not gpu", "-p", "no:cacheprovider"], env=env, cwd=ROOT, capture_output=True,
                       text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-3000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-3000:]
