"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): api.cpp is compiled with the sanitizers on its host pass, linked
with the library's other objects into tests/host_abi_driver.c, and the driver
calls every entry point with arguments that the host checks must reject."""

import os
import shutil
import subprocess

import pytest

from long_context_decode_microattention_amd import build as da_build

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
OUT = os.path.join(ROOT, "_build", "host_sanitizers")
# host pass only: the device code is built exactly as in the library
SAN = ["address", "undefined"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


@pytest.fixture(scope="module")
def driver():
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    if not os.path.exists(da_build.LIB_PATH):
        da_build.build()
    os.makedirs(OUT, exist_ok=True)
    api = os.path.join(da_build.CSRC, "api.cpp")
    api_obj = os.path.join(OUT, "api_sanitized.o")
    host_san = []
    for s in SAN:
        host_san += ["-Xarch_host", f"-fsanitize={s}"]
    host_san += ["-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    _run([da_build.hipcc(), "-x", "hip", *da_build.COMMON_FLAGS, *host_san, "-c", api, "-o", api_obj])
    drv_obj = os.path.join(OUT, "driver.o")
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(da_build.hipcc())))
    san = [f"-fsanitize={','.join(SAN)}", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
    _run(["gcc", "-std=c11", "-g", "-O1", *san, "-D__HIP_PLATFORM_AMD__", "-I", da_build.INCLUDE,
          "-I", os.path.join(rocm, "include"), "-c", os.path.join(HERE, "host_abi_driver.c"),
          "-o", drv_obj])
    others = [os.path.join(da_build.BUILD_DIR, os.path.basename(s) + ".o")
              for s in da_build.sources() if not s.endswith("api.cpp")]
    missing = [o for o in others if not os.path.exists(o)]
    if missing:
        da_build.build()
    exe = os.path.join(OUT, "host_abi_driver")
    _run(["g++", *san, drv_obj, api_obj, *others, "-L", os.path.join(rocm, "lib"),
          f"-Wl,-rpath,{os.path.join(rocm, 'lib')}", "-lamdhip64", "-o", exe])
    return exe


def test_host_abi_under_sanitizers(driver):
    env = dict(os.environ)
    # leak reports would cover the HIP runtime's own start-up allocations;
    # another preloaded library may precede the sanitizer runtime
    env["ASAN_OPTIONS"] = "detect_leaks=0:verify_asan_link_order=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([driver], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, f"exit {r.returncode}\n{r.stdout}\n{r.stderr[-4000:]}"
    assert "host ABI checks passed" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
