"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

Every source of libagnes_gdn is rebuilt with the host pass instrumented (the device code is
built as usual and never runs here), and tests/sanitize/abi_checks.cpp, built with the same
sanitizers, drives every C-ABI entry point through its argument checks: the ordinary rejects
and the extremes of every size, stride and count.  A sanitizer report aborts the driver, and
any status other than the expected one fails it.
"""
import concurrent.futures as cf
import os
import shutil
import subprocess

import pytest

from gated_delta_rule_35_amd import build as libbuild

HERE = os.path.dirname(os.path.abspath(__file__))
DRIVER = os.path.join(HERE, "sanitize", "abi_checks.cpp")
CLANG = "/opt/rocm/llvm/bin/clang++"
# Each sanitizer flag goes to the host pass only: the device code is compiled unchanged.
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]
DRIVER_SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    if r.returncode != 0:
        raise RuntimeError(f"{' '.join(cmd[:3])} ... failed ({r.returncode}):\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}")
    return r


@pytest.fixture(scope="module")
def sanitized_driver(tmp_path_factory):
    if not (os.path.exists(CLANG) and shutil.which("hipcc") or os.path.exists("/opt/rocm/bin/hipcc")):
        pytest.skip("the ROCm toolchain is not installed")
    out = tmp_path_factory.mktemp("san")
    hipcc = libbuild._hipcc()
    inc = ["-I", os.path.join(libbuild.ROOT, "include"), "-I", libbuild.CSRC]

    def compile_one(src):
        obj = os.path.join(out, os.path.basename(src) + ".o")
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        _run([hipcc, *lang, *libbuild.HIP_FLAGS, *HOST_SAN, *inc, "-c", src, "-o", obj])
        return obj

    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(compile_one, libbuild.sources()))
    lib = os.path.join(out, "libagnes_gdn_san.so")
    _run([hipcc, f"--offload-arch={libbuild.ARCH}", "-shared", "-fPIC", *objs, "-o", lib])
    exe = os.path.join(out, "abi_checks")
    _run([CLANG, "-std=c++17", "-O1", *DRIVER_SAN, *inc, DRIVER, lib, f"-Wl,-rpath,{out}", "-o", exe])
    return exe


def test_abi_checks_under_asan_and_ubsan(sanitized_driver):
    env = dict(os.environ)
    # The HIP runtime keeps its process-lifetime objects to the end: leak checking is off, every
    # other ASan check and every UBSan check aborts the run at the first report.
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:verify_asan_link_order=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([sanitized_driver], capture_output=True, text=True, env=env, timeout=300)
    report = r.stdout + r.stderr
    assert r.returncode == 0, report[-6000:]
    assert "runtime error" not in report and "AddressSanitizer" not in report, report[-6000:]
    assert "all passed" in r.stdout
