"""The host code of the C ABI (argument validation, workspace sizing, kernel
selection) built with AddressSanitizer and UndefinedBehaviorSanitizer and
driven through every entry point's paths (tests/host_sanitize/driver.cpp).

The sanitizers instrument the host side only (each -fsanitize= after
-Xarch_host); the device code is built as usual.  The run hides every GPU,
so no kernel can launch and calls that pass validation end in
SPA_ERR_LAUNCH; the driver's device pointers are fake and never
dereferenced."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_paged_attention_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _hipcc():
    return shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def test_host_code_under_asan_and_ubsan(tmp_path):
    from sparse_paged_attention_amd import build as b
    if not os.path.exists(_hipcc()):
        pytest.skip("hipcc not available")
    objs = []
    for src in b.SOURCES:      # device code as in the library; host code instrumented
        obj = str(tmp_path / (os.path.splitext(src)[0] + ".o"))
        cmd = [_hipcc(), "-c", "-x", "hip", "-O1", "-g", "-std=c++17", "-fPIC",
               f"--offload-arch={b.ARCH}", "-I", INCLUDE, "-I", CSRC, os.path.join(CSRC, src), "-o", obj] + SAN + \
              b.DEVICE_FLAGS + b.SOURCE_FLAGS.get(src, [])
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        objs.append(obj)
    drv = str(tmp_path / "driver.o")
    r = subprocess.run([_hipcc(), "-c", "-x", "hip", "-O1", "-g", "-std=c++17",
                        f"--offload-arch={b.ARCH}", "-I", INCLUDE, os.path.join(ROOT, "tests", "host_sanitize",
                                                                                  "driver.cpp"), "-o", drv] + SAN,
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    exe = str(tmp_path / "driver")
    clang = "/opt/rocm/llvm/bin/clang++"
    link = [clang, "-fsanitize=address,undefined", drv] + objs + ["-L/opt/rocm/lib", "-lamdhip64",
                                                                   "-Wl,-rpath,/opt/rocm/lib", "-o", exe]
    r = subprocess.run(link, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1", CUDA_VISIBLE_DEVICES="-1",
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-4000:]
    assert r.returncode == 0, (r.stdout, r.stderr[-4000:])
    assert "0 unexpected statuses" in r.stdout
