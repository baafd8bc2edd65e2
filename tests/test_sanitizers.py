"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two rebuilds, each loaded into a child process whose sanitizer runtime is
preloaded (Python itself is not instrumented, so leak reports are off):

* the C oracle and the host generator (gcc), running the oracle pin suites;
* the host half of the HIP library (hipcc, device code built as usual and
  not instrumented), running the C-ABI checks that need no GPU: symbol
  export, workspace sizes and their overflow guards, status strings and
  every argument rejection before a launch.

Any sanitizer report aborts the child, which fails the test.
"""
import glob
import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}
GCC_SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r


def _plugin(tmp, body):
    """A pytest plugin module that repoints the libraries before any test."""
    path = os.path.join(tmp, "san_libs.py")
    with open(path, "w") as f:
        f.write(textwrap.dedent(body))
    return tmp


def _pytest_child(tmp, preload, files, extra=()):
    env = dict(os.environ, **SAN_ENV, LD_PRELOAD=preload,
               PYTHONPATH=os.pathsep.join([tmp, ROOT, os.path.join(ROOT, "tests")]))
    env.pop("PYTEST_ADDOPTS", None)
    return _run([sys.executable, "-m", "pytest", "-q", "-p", "san_libs", "-m", "not gpu",
                 "-p", "no:cacheprovider", *extra, *[os.path.join(ROOT, "tests", f) for f in files]],
                env=env, cwd=tmp, timeout=900)


def test_oracle_and_generator_under_asan_ubsan(tmp_path):
    tmp = str(tmp_path)
    rt = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                        text=True).stdout.strip()
    if not os.path.isabs(rt) or not os.path.exists(rt):
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    ora = os.path.join(tmp, "liboracle_san.so")
    gen = os.path.join(tmp, "libsynth_cpu_san.so")
    _run(["gcc", *GCC_SAN, "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
          "-o", ora, os.path.join(ROOT, "oracle", "drgrpo_oracle.c"), "-lm"])
    _run(["gcc", *GCC_SAN, "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared", "-o", gen,
          os.path.join(ROOT, "synth", "synth_cpu.c")])
    _plugin(tmp, f"""
        import oracle, synth
        def pytest_configure(config):
            oracle.LIB, oracle._lib = {ora!r}, None
            synth.CPU_LIB, synth._cpu = {gen!r}, None
        """)
    r = _pytest_child(tmp, rt, ["test_oracle_pins.py", "test_oracle_variants.py"])
    assert " passed" in r.stdout and "failed" not in r.stdout, r.stdout[-2000:]


def test_library_host_code_under_asan_ubsan(tmp_path):
    tmp = str(tmp_path)
    rts = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not rts:
        pytest.skip("the ROCm compiler's AddressSanitizer runtime is not installed")
    from rl_post_loss_dr_amd.build import HIPCC_FLAGS, SOURCES

    lib = os.path.join(tmp, "libdrgrpo_san.so")
    # sanitizers on the host half only: each -fsanitize flag goes to the host
    # compilation through -Xarch_host
    host = []
    for flag in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all",
                 "-fno-omit-frame-pointer", "-g"):
        host += ["-Xarch_host", flag]
    flags = [f if f != "-O3" else "-O1" for f in HIPCC_FLAGS]
    _run(["hipcc", *flags, *host, "-shared-libsan", "-I", os.path.join(ROOT, "include"),
          "-o", lib, *SOURCES], timeout=900)
    _plugin(tmp, f"""
        import rl_post_loss_dr_amd as dr
        def pytest_configure(config):
            dr.LIB, dr._lib = {lib!r}, None
        """)
    r = _pytest_child(tmp, rts[0], ["test_abi.py"],
                      extra=["-k", "not graft_entry_build and not ceiling_library"])
    assert " passed" in r.stdout and "failed" not in r.stdout, r.stdout[-2000:]
