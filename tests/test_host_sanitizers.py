"""The library's host code under AddressSanitizer, LeakSanitizer and
UndefinedBehaviorSanitizer, on the CPU: every source is compiled with the
sanitizers on its host side only (the device code is built as usual and never
runs), linked into the C driver tests/host/abi_sanitize.c, and run.  The
driver covers config checks and sizing, argument checks, NULL handles, the
per-thread error message and (with no device present) the clean-up of a
create that fails at its first runtime call."""

import os
import shlex
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "quantized_moe_expert_gemv_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
DRIVER = os.path.join(ROOT, "tests", "host", "abi_sanitize.c")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang")
SOURCES = ["strata_moe.hip", "repack.hip", "decode.hip", "prefill.hip"]

# host-side sanitizers only: each one right after -Xarch_host
HOST_SAN = shlex.split("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
                       "-Xarch_host -fno-omit-frame-pointer -Xarch_host -fno-sanitize-recover=all")

pytestmark = pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)),
                                reason="hipcc / clang not found")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    d = tmp_path_factory.mktemp("asan")
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             *HOST_SAN, "-I", INCLUDE, "-I", CSRC]
    objs = [str(d / s.replace(".hip", ".o")) for s in SOURCES]
    jobs = [[HIPCC, *flags, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
    with ThreadPoolExecutor(max_workers=4) as ex:
        list(ex.map(_run, jobs))
    drv_o = str(d / "abi_sanitize.o")
    san = "-fsanitize=address,undefined"
    _run([CLANG, "-g", "-O1", "-std=c11", "-Wall", "-Werror", san, "-fno-sanitize-recover=all",
          "-I", INCLUDE, "-c", DRIVER, "-o", drv_o])
    exe = str(d / "abi_sanitize")
    _run([CLANG + "++", san, drv_o, *objs, "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
          "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-lpthread", "-o", exe])
    return exe


def test_host_code_is_clean_under_asan_lsan_ubsan(driver):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:exitcode=23",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1:exitcode=24")
    r = subprocess.run([driver], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, f"rc {r.returncode}\n{r.stdout}\n{r.stderr[-4000:]}"
    assert r.stdout.startswith("ok "), r.stdout
    assert "runtime error" not in r.stderr and "Sanitizer" not in r.stderr, r.stderr[-4000:]
    assert int(r.stdout.split()[1]) > 1000
