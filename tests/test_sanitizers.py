"""Address and undefined-behaviour sanitizers on the CPU code.

* The oracle (plain C) is rebuilt with -fsanitize=address,undefined and the
  oracle's pin tests (tests/test_oracle.py) run against that build.
* The C ABI's host code (csrc/api.cpp: argument validation, segment tables,
  kernel choice) is rebuilt with the same sanitizers on the host side only
  and linked with the ordinary device objects; the ABI tests
  (tests/test_abi.py, every call rejected before any HIP call) run against
  that library.

Each run is a child Python process with the sanitizer runtime preloaded;
any sanitizer report fails the run (halt_on_error).  Skipped where the
environment already preloads a library of its own, or where a GPU is present
(the ABI tests pass fake device pointers and run only without one)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

SAN_DIR = os.path.join(ROOT, "segmented_dual_scale_amd", "_build", "sanitize")

pytestmark = pytest.mark.skipif(bool(os.environ.get("LD_PRELOAD")),
                                reason="the environment preloads a library of its own")


def _gpu_present():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def _run_pytest(test_file: str, preload: str, env_extra: dict) -> subprocess.CompletedProcess:
    env = dict(os.environ)
    env.update(env_extra)
    env["LD_PRELOAD"] = preload
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
           "-m", "not gpu", os.path.join(ROOT, "tests", test_file)]
    return subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)


def _check(r: subprocess.CompletedProcess, what: str):
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out, out[-4000:]
    assert "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, f"{what} under sanitizers failed (rc {r.returncode}):\n{out[-4000:]}"
    assert " passed" in out, out[-2000:]


def test_oracle_pins_under_asan_ubsan():
    os.makedirs(SAN_DIR, exist_ok=True)
    lib = os.path.join(SAN_DIR, "liboracle_asan_ubsan.so")
    src = os.path.join(ROOT, "oracle", "segquant_oracle.c")
    subprocess.run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
                    "-o", lib, src, "-lm"], check=True)
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True, check=True).stdout.strip()
    r = _run_pytest("test_oracle.py", asan, {"SEGQUANT_ORACLE_LIBRARY": lib})
    _check(r, "tests/test_oracle.py")


@pytest.mark.skipif(_gpu_present(), reason="the ABI tests pass fake device pointers: CPU only")
def test_abi_validation_under_asan_ubsan():
    from segmented_dual_scale_amd import build as B
    os.makedirs(SAN_DIR, exist_ok=True)
    # host-only instrumentation: every -fsanitize goes to the host pass
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]
    api_obj = B.compile_source("api.cpp", out=os.path.join(SAN_DIR, "api_asan_ubsan.o"),
                               extra_flags=san)
    objs = []
    for src in B.SOURCES:
        if src == "api.cpp":
            continue
        o = B.object_path(src)
        if not os.path.exists(o):
            B.compile_source(src)
        objs.append(o)
    lib = B.link_shared(os.path.join(SAN_DIR, "libsegquant_asan_ubsan.so"), [api_obj, *objs],
                        ["-Xarch_host", "-fsanitize=address", "-Xarch_host",
                         "-fsanitize=undefined", "-shared-libsan"])
    clang_rt = subprocess.run([B._hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"],
                              capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(clang_rt) or not os.path.exists(clang_rt):
        import glob
        found = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
        assert found, "clang's address-sanitizer runtime not found"
        clang_rt = found[0]
    r = _run_pytest("test_abi.py", clang_rt, {"SEGQUANT_LIBRARY": lib})
    _check(r, "tests/test_abi.py")
