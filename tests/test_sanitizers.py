"""The CPU oracle and the host side of libp3d under the sanitizers (CPU
only, no device work).

1. The oracle's C source is built with AddressSanitizer and UBSan (gcc,
   -fno-sanitize-recover: the first report aborts) and every oracle pin,
   the whole-path composition among them, runs against that build in a
   child process with the ASan runtime preloaded.
2. libp3d is built with AddressSanitizer on the host code only (device code
   is compiled normally and never runs here) and the C-ABI tests -- every
   argument check of every entry point, the host helpers and the figures --
   run against that build.
Both children verify that the sanitized library is the one they loaded.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

# host-side sanitizer flags for hipcc: each -fsanitize= goes to the host
# compilation only
HOST_ASAN = "-Xarch_host -fsanitize=address -Xarch_host -fno-omit-frame-pointer".split()


def _gcc_runtime(name):
    path = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True,
                          check=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _clang_asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def _run_child(code, env, timeout=900):
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=timeout)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-6000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-6000:]
    return out


def test_sanitizer_runtime_catches_a_planted_overflow(tmp_path):
    """The toolchain check: a one-past-the-end read in a tiny C library built
    the same way is reported, so a clean run below means something."""
    asan = _gcc_runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc has no AddressSanitizer runtime")
    src = tmp_path / "planted.c"
    src.write_text("#include <stdlib.h>\n"
                   "int planted(int n) { int* p = malloc(n * sizeof(int));\n"
                   "  for (int i = 0; i < n; ++i) p[i] = i;\n"
                   "  int v = p[n]; free(p); return v; }\n")
    lib = tmp_path / "libplanted.so"
    subprocess.run(["gcc", "-O1", "-fPIC", "-shared", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", str(src), "-o", str(lib)], check=True)
    env = dict(os.environ, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0")
    r = subprocess.run([sys.executable, "-c",
                        "import ctypes; ctypes.CDLL(%r).planted(8)" % str(lib)],
                       env=env, capture_output=True, text=True, timeout=120)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr


def test_oracle_pins_under_asan_ubsan(tmp_path):
    asan = _gcc_runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc has no AddressSanitizer runtime")
    from oracle import build as obuild
    lib = obuild.build(out=str(tmp_path / "liboracle_asan.so"),
                       extra=["-O1", "-g", "-fno-omit-frame-pointer",
                              "-fsanitize=address,undefined", "-fno-sanitize-recover=all"])
    env = dict(os.environ, P3D_ORACLE_LIB=lib, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="4")
    out = _run_child(
        "import sys, oracle\n"
        "assert oracle.get().path == %r, oracle.get().path\n"
        "import pytest\n"
        "sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', 'tests/test_oracle_pins.py']))\n"
        % lib, env)
    import oracle_pins
    assert "whole_path_composition" in oracle_pins.ALL_PINS
    assert "%d passed" % len(oracle_pins.ALL_PINS) in out, out[-2000:]


def test_abi_under_host_asan(tmp_path):
    rt = _clang_asan_runtime()
    if rt is None:
        pytest.skip("no clang AddressSanitizer runtime under /opt/rocm/llvm")
    from pixel_aligned_image_amd import build as pbuild
    lib = pbuild.build(out=str(tmp_path / "libp3d_hostasan.so"), objdir=str(tmp_path / "obj"),
                       extra=["-O1", "-g0", "-Xarch_host", "-g", *HOST_ASAN],
                       link_extra=HOST_ASAN[:2])
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True, check=True).stdout
    assert "__asan_report" in syms, "host code is not instrumented"
    env = dict(os.environ, P3D_LIB=lib, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0")
    out = _run_child(
        "import sys, pixel_aligned_image_amd as p\n"
        "assert p.LIB_PATH == %r, p.LIB_PATH\n"
        "import pytest\n"
        "sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', 'tests/test_abi.py']))\n" % lib,
        env)
    assert " passed" in out
