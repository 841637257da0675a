"""The C ABI's argument validation under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU: the host part of the ABI layer
(csrc/api.hip) is rebuilt with both sanitizers on its host code only, linked
with the library's kernel objects, and driven through every entry point by a
small C program (tests/sanitize/abi_driver.c) with arguments the library must
refuse, so only validation and error reporting run."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "separator_kv_cache_amd")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"
# each sanitizer flag applies to host code only (the device code is built as usual)
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm toolchain not found")
def test_abi_validation_under_address_and_ub_sanitizers(tmp_path):
    sys.path.insert(0, ROOT)
    from separator_kv_cache_amd import build as b
    objs = [os.path.join(b.OBJ, s.replace(".hip", ".o")) for s in b.SOURCES if s != "api.hip"]
    if not all(os.path.exists(o) for o in objs):
        b.build(jobs=4)
    api_o = str(tmp_path / "api_san.o")
    _run([HIPCC, "-O1", "-g", "-std=c++17", "-fPIC", "-fvisibility=hidden", "--offload-arch=gfx950",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument",
          *HOST_SAN, "-I", os.path.join(ROOT, "include"), "-c", os.path.join(PKG, "csrc", "api.hip"), "-o", api_o])
    lib = str(tmp_path / "libsepattn_san.so")
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-shared-libsan", *HOST_SAN,
          "-o", lib, api_o, *objs])
    rt = subprocess.run([CLANG, "-print-resource-dir"], capture_output=True, text=True).stdout.strip()
    rt_lib = os.path.join(rt, "lib", "linux")  # the sanitizer runtimes
    exe = str(tmp_path / "abi_driver")
    _run([CLANG, "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-shared-libsan",
          "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "sanitize", "abi_driver.c"),
          lib, f"-Wl,-rpath,{tmp_path}", f"-Wl,-rpath,{rt_lib}", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and "ok: 0 unexpected" in r.stdout, f"{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-3000:]
