"""The C ABI's host validation under AddressSanitizer and UndefinedBehaviorSanitizer.

The library's sources are compiled for gfx950 with the host half instrumented by both sanitizers
(the device code is built as usual; nothing here launches it, so no GPU is needed), and linked with
`tests/sanitize_validation.cpp`, a driver that drives every entry point's validation to its edges (group counts, negative and huge split sizes,
32-bit extents, widths, NULL pointers, enum values, short workspaces, device-resident split sizes,
the allocation-free backward's scratch limit) and checks each returned code.  Any out-of-bounds
access, use of uninitialised stack memory caught by ASan, signed overflow, shift or conversion
error aborts the driver with a sanitizer report.  Two planted faults in the driver (a heap read
past the end, a signed overflow) show that both sanitizers are live in the build.
"""

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "moe_grouped_scaled_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang++"
SOURCES = ["mgs_api.hip", "act_quant.hip", "gemm_mx.hip"]


def _run(cmd, **kw):
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, **kw)
    return res.returncode, res.stdout


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="needs the ROCm toolchain")
def test_validation_layer_is_clean_under_asan_and_ubsan(tmp_path):
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    objs = [str(tmp_path / src.replace(".hip", ".o")) for src in SOURCES]

    def compile_one(i):
        return _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", *san,
                     "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                     "-I", os.path.join(ROOT, "include"), "-c", os.path.join(CSRC, SOURCES[i]), "-o", objs[i]])

    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        for rc, out in ex.map(compile_one, range(len(SOURCES))):
            assert rc == 0, out
    drv = str(tmp_path / "drv.o")
    rc, out = _run([CLANG, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
                    "-c", os.path.join(ROOT, "tests", "sanitize_validation.cpp"), "-o", drv])
    assert rc == 0, out
    exe = str(tmp_path / "validate")
    rc, out = _run([HIPCC, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
                    "-fsanitize=undefined", "-o", exe, drv, *objs, "-Wl,-rpath,/opt/rocm/lib"])
    assert rc == 0, out
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    rc, out = _run([exe], env=env, timeout=300)
    print(out)
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out
    assert rc == 0, out
    assert " 0 failed" in out
    rc, out = _run([exe, "oob"], env=env, timeout=60)
    assert rc != 0 and "heap-buffer-overflow" in out, out
    rc, out = _run([exe, "overflow"], env=env, timeout=60)
    assert rc != 0 and "signed integer overflow" in out, out
