"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* oracle.c built with gcc -fsanitize=address,undefined, and the oracle's pin tests run
  against that build (ORACLE_LIB) in a child process with the ASan runtime preloaded.
* The C ABI's host side (capi.cpp, step.cpp: every argument check, workspace sizing, the
  step descriptor) compiled host-only by hipcc with the sanitizers on the host pass, linked
  with the kernels' objects of the normal build, and the host ABI tests run against that
  library (CTR_LIB) the same way.  No device code is instrumented and no GPU is used.

Both builds abort on the first report (-fno-sanitize-recover=all), so a clean child exit with
every test passed means no report.  Leak checking is off: the interpreter keeps its objects
until exit by design.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
BUILD = os.path.join(ROOT, "sparse_embedding_lookup_amd", "_build")
CSRC = os.path.join(ROOT, "sparse_embedding_lookup_amd", "csrc")
SAN_OPTS = {
    "ASAN_OPTIONS": "detect_leaks=0:alloc_dealloc_mismatch=0:detect_odr_violation=0:"
                    "verify_asan_link_order=0:abort_on_error=1",
    "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
}


def _run_pytest(files, env_extra, preload):
    env = dict(os.environ)
    env.update(SAN_OPTS)
    env.update(env_extra)
    env["LD_PRELOAD"] = preload
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu"] + files, cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out, out[-2000:]
    return out


def _instrumented(path):
    syms = subprocess.run(["nm", "-D", "--undefined-only", path], capture_output=True,
                          text=True, check=True).stdout
    return "__asan_report" in syms and "__ubsan_handle" in syms


def test_oracle_under_asan_and_ubsan(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.check_call(["gcc", "-std=c11", "-O1", "-g", "-ffp-contract=off", "-fno-fast-math",
                           "-fopenmp", "-fPIC", "-shared", "-fno-omit-frame-pointer",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                           "-o", lib, os.path.join(ROOT, "oracle", "oracle.c"), "-lm"])
    assert _instrumented(lib)
    runtime = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                             text=True, check=True).stdout.strip()
    tests = sorted(glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py")))
    out = _run_pytest(tests, {"ORACLE_LIB": lib}, runtime)
    print(out.strip().splitlines()[-1])


def test_capi_host_under_asan_and_ubsan(tmp_path):
    objs = [os.path.join(BUILD, f + ".o") for f in
            ("unique.hip", "embbag.hip", "segreduce.hip", "interaction.hip", "dict.hip",
             "dense.hip", "fused.hip")]
    if not os.path.exists(HIPCC) or not all(os.path.exists(o) for o in objs):
        pytest.skip("needs hipcc and the kernels' objects of the normal build")
    runtimes = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not runtimes:
        pytest.skip("no clang ASan runtime")
    host_flags = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=all"]
    san_objs = []
    for src in ("capi.cpp", "step.cpp"):
        o = str(tmp_path / (src + ".o"))
        subprocess.check_call([HIPCC, "-x", "hip", "--offload-arch=gfx950", "--cuda-host-only",
                               "-std=c++17", "-O1", "-g", "-fPIC", "-fno-omit-frame-pointer",
                               "-Wno-unused-command-line-argument"] + host_flags +
                              ["-c", os.path.join(CSRC, src), "-o", o])
        san_objs.append(o)
    lib = str(tmp_path / "libctr_san.so")
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-shared-libsan"] +
                          host_flags[:4] + ["-o", lib] + san_objs + objs)
    assert _instrumented(lib)
    out = _run_pytest([os.path.join(ROOT, "tests", "test_capi_host.py")], {"CTR_LIB": lib},
                      runtimes[0])
    print(out.strip().splitlines()[-1])
