"""The C ABI's host layer under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds the library with both sanitizers on the host pass (device code as
usual), then runs the CPU boundary and binding tests in a child process that
preloads the ASan runtime and loads that build.  Every call there is rejected
by argument validation before any HIP call, so the run needs no GPU; an
out-of-bounds read of a segment table, an overflowing size product or a
misaligned access in the checks would end the child with a sanitizer report.
"""

import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


@pytest.fixture(scope="module")
def san_env(tmp_path_factory):
    from streaming_diffusion_portrait_amd import build as Bld
    try:
        Bld._hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("clang ASan runtime not found")
    d = tmp_path_factory.mktemp("san")
    lib = Bld.build(sanitize=True, lib_path=str(d / "libpl_san.so"), obj_dir=str(d / "obj"))
    env = dict(os.environ)
    pre = env.get("LD_PRELOAD", "")
    env["LD_PRELOAD"] = rt + (":" + pre if pre else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["PL_LIBRARY"] = lib
    env["PYTHONPATH"] = ROOT + (os.pathsep + env["PYTHONPATH"] if env.get("PYTHONPATH") else "")
    return env, lib


def test_sanitized_build_is_the_one_loaded(san_env):
    env, lib = san_env
    code = ("from streaming_diffusion_portrait_amd import binding as B; B.load(); "
            "maps = open('/proc/self/maps').read(); "
            "print('san-lib' if B.LIB_PATH in maps else 'other-lib', "
            "'asan-rt' if 'libclang_rt.asan' in maps else 'no-rt')")
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-4000:]
    assert r.stdout.split() == ["san-lib", "asan-rt"], r.stdout


def test_boundary_checks_run_clean_under_sanitizers(san_env):
    env, _ = san_env
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_boundary.py"),
                        os.path.join(ROOT, "tests", "test_binding_checks.py")],
                       env=env, capture_output=True, text=True, timeout=600, cwd=ROOT)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-6000:]
    assert "runtime error" not in out, out[-6000:]
    assert r.returncode == 0, out[-6000:]
    assert " passed" in out and " failed" not in out, out[-2000:]
