"""Host-side AddressSanitizer + UndefinedBehaviorSanitizer runs (CPU only).

The CPU oracle (oracle/hs2_oracle.c) and the host half of the library's C ABI
(hs2_api.cpp: validation, workspace layout, chunk fitting, the varlen task
planner) are rebuilt with -fsanitize=address,undefined by gcc/g++ (the GPU
kernels' objects are linked unchanged: device code is not instrumented), and
the oracle pins and the C ABI tests are rerun against those builds in a child
process with the ASan runtime preloaded. Any out-of-bounds access, use after
free or undefined behaviour in that host code fails the run.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "token_level_sparse_hs2_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
       "-fno-omit-frame-pointer", "-g", "-O1"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r


@pytest.fixture(scope="module")
def sanitized_libs(tmp_path_factory):
    from token_level_sparse_hs2_amd import _build
    out = tmp_path_factory.mktemp("asan")
    oracle_so = str(out / "libhs2_oracle_asan.so")
    _run(["gcc", *SAN, "-std=c11", "-fPIC", "-shared", "-pthread",
          os.path.join(ROOT, "oracle", "hs2_oracle.c"), "-o", oracle_so, "-lm"])
    # the kernels' objects as the normal build makes them
    kernel_objs = [os.path.join(_build.BUILD_DIR, s + ".o") for s in _build.SOURCES
                   if s.endswith(".hip")]
    if not all(os.path.exists(o) for o in kernel_objs):
        _build.build()
    api_o = str(out / "hs2_api_asan.o")
    _run(["g++", *SAN, "-std=c++17", "-fPIC", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
          f"-I{_build.INCLUDE}", f"-I{CSRC}", "-c", os.path.join(CSRC, "hs2_api.cpp"), "-o", api_o])
    lib_so = str(out / "libhs2_asan.so")
    _run(["g++", "-shared", "-fsanitize=address,undefined", api_o, *kernel_objs,
          "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", lib_so])
    return oracle_so, lib_so


def test_oracle_and_host_abi_under_asan_ubsan(sanitized_libs):
    oracle_so, lib_so = sanitized_libs
    asan_rt = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                             text=True).stdout.strip()
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": asan_rt,
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:exitcode=97",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1:exitcode=98",
        "HS2_ORACLE_LIB": oracle_so,
        "HS2_LIBRARY": lib_so,
    })
    # the child loads the sanitized builds (and the ASan runtime), not the normal ones
    probe = ("import oracle, token_level_sparse_hs2_amd as h; oracle._load(); h.load_library(); "
             "print(open('/proc/self/maps').read())")
    maps = _run([sys.executable, "-c", probe], env=env, cwd=ROOT).stdout
    assert oracle_so in maps and lib_so in maps and "libasan" in maps
    tests = [os.path.join(ROOT, "tests", f) for f in ("test_oracle_pins.py", "test_abi_cpu.py")]
    r = subprocess.run([sys.executable, "-m", "pytest", *tests, "-q", "-x", "-m", "not gpu",
                        "-p", "no:cacheprovider"], capture_output=True, text=True, env=env,
                       cwd=ROOT, timeout=1500)
    tail = (r.stdout[-3000:] + "\n" + r.stderr[-6000:])
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, tail
