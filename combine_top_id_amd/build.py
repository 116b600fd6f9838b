"""Builds libmoonep.so (the hot path) and libmoonep_streams.so (the memory streams the
benchmark measures ceilings with) for gfx950 with hipcc, in-tree next to this file."""

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = ["moonep_api.hip", "moonep_plan.hip", "moonep_move.hip"]
STREAM_SOURCES = ["moonep_streams.hip"]

HIPCC_FLAGS = [
    "-O3", "--offload-arch=gfx950", "-std=c++17", "-fPIC", "-shared",
    # combine and reduce round each fp32 product and sum separately
    "-ffp-contract=off",
    # no packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _hipcc(sources, name, verbose):
    out = os.path.join(HERE, name)
    tmp = out + ".tmp"
    cmd = ["/opt/rocm/bin/hipcc", *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(HERE, "csrc"),
           *[os.path.join(HERE, "csrc", f) for f in sources], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + r.stderr[-4000:])
    os.replace(tmp, out)
    return out


def build(verbose=False):
    out = _hipcc(SOURCES, "libmoonep.so", verbose)
    _hipcc(STREAM_SOURCES, "libmoonep_streams.so", verbose)
    build_c_smoke(verbose)
    return out


def build_c_smoke(verbose=False):
    """A plain C consumer of the C ABI (tests/c_abi/smoke.c), linked against the library
    just built; the library is found next to it through a relative run path."""
    src = os.path.join(ROOT, "tests", "c_abi", "smoke.c")
    out = os.path.join(ROOT, "tests", "c_abi", "smoke")
    cmd = ["gcc", "-std=c11", "-O1", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", "/opt/rocm/include", src, "-L", HERE, "-lmoonep", "-L", "/opt/rocm/lib",
           "-lamdhip64", "-Wl,-rpath,$ORIGIN/../../combine_top_id_amd",
           "-Wl,-rpath,/opt/rocm/lib", "-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("gcc failed:\n" + r.stderr[-4000:])
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
