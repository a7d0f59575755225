"""The library's host code (argument checks and launch planning of every C-ABI
entry point) and the input generator, built with AddressSanitizer and
UndefinedBehaviorSanitizer on the host side only (device code is not
instrumented) and run on a host without a GPU by tests/sanitize/host_driver.cpp:
invalid descriptors, extreme sizes, NULL and misaligned pointers, workspace
sizes at their limits, status texts and the generator's streams and rounding.
Any sanitizer finding aborts the driver."""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "kv_cache_eviction_lse_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"
LIB_SOURCES = ["api.cpp", "lse.hip", "score.hip", "evict.hip", "attn.hip", "vnorm.hip", "decode.hip", "stream.hip"]
# sanitizers on the host pass only: each -fsanitize= after -Xarch_host
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
C_SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(ln for ln in (r.stdout + r.stderr).splitlines() if noise not in ln)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{msgs}"


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="needs the ROCm toolchain")
def test_host_code_under_asan_and_ubsan(tmp_path):
    def lib_obj(src):
        out = str(tmp_path / (os.path.splitext(src)[0] + ".o"))
        _run([HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *HOST_SAN, "-c",
              os.path.join(CSRC, src), "-o", out])
        return out

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lib_obj, LIB_SOURCES))
    gen = str(tmp_path / "gen.o")
    _run([CLANG, "-O1", "-g", *C_SAN, "-c", os.path.join(ROOT, "synth", "gen.c"), "-o", gen])
    drv = str(tmp_path / "drv.o")
    _run([CLANG + "++", "-O1", "-g", "-std=c++17", *C_SAN, "-I", os.path.join(ROOT, "include"), "-c",
          os.path.join(ROOT, "tests", "sanitize", "host_driver.cpp"), "-o", drv])
    exe = str(tmp_path / "host_driver")
    _run([HIPCC, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
          drv, gen, *objs, "-o", exe])
    env = dict(os.environ)
    # the HIP runtime keeps allocations until exit; leak reports are not the point here
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["HIP_VISIBLE_DEVICES"] = ""  # (stay off any GPU: valid calls must stop at KVS_ENODEV)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "all expectations met" in out, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    shutil.rmtree(tmp_path, ignore_errors=True)
