"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Builds the library sources with both sanitizers on the host side only (each -fsanitize=
flag behind -Xarch_host; the device code is compiled as usual and never runs here), links
them with tests/c_abi/asan_host.c and runs it.  Every call that driver makes returns from
its host-side argument checks before any HIP call, so no GPU is needed: it covers
moonep_query over a sweep of sizes (limits and int32 overflow included), every entry
point's argument-error paths, moonep_strerror, and the stream library's checks.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "combine_top_id_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
SOURCES = ["moonep_api.hip", "moonep_plan.hip", "moonep_move.hip", "moonep_streams.hip"]


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)),
                    reason="needs the ROCm toolchain")
def test_c_abi_host_paths_under_sanitizers(tmp_path):
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    procs, objs = [], []
    for src in SOURCES:
        obj = str(tmp_path / (src + ".o"))
        objs.append(obj)
        cmd = [HIPCC, "-O1", "--offload-arch=gfx950", "-std=c++17", "-fPIC", "-c",
               "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
               "-Xarch_host", "-fno-omit-frame-pointer", *inc, os.path.join(CSRC, src), "-o", obj]
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE,
                                            text=True)))
    for src, p in procs:
        out, err = p.communicate(timeout=600)
        assert p.returncode == 0, f"{src}:\n{err[-3000:]}"
    # the C driver and the link are host-only steps (plain clang, no HIP sources)
    drv = str(tmp_path / "asan_host.o")
    host_san = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer"]
    r = subprocess.run([CLANG, "-O1", "-g", "-std=c11", *host_san, "-D__HIP_PLATFORM_AMD__",
                        "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include", "-c",
                        os.path.join(ROOT, "tests", "c_abi", "asan_host.c"), "-o", drv],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    exe = str(tmp_path / "asan_host")
    r = subprocess.run([CLANG + "++", *host_san, drv, *objs, "-L/opt/rocm/lib", "-lamdhip64",
                        "-Wl,-rpath,/opt/rocm/lib", "-o", exe],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0 and "asan host ok" in r.stdout, r.stdout[-3000:] + r.stderr[-3000:]
