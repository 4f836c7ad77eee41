"""Build libkvc.so (HIP, gfx950) in place.

    python -m compressed_kv_cache_compress_amd.build

One hipcc invocation compiles the host planner and the kernels into a shared
library with a plain C ABI (include/kvc.h).  Flags that matter for
correctness:
  -ffp-contract=off                      no implicit fma contraction (the
                                         selection path's fp32 sequence is
                                         specified operation by operation)
  -fno-gpu-flush-denormals-to-zero       IEEE fp32 denormals
  -target-feature -packed-fp32-ops       no packed fp32 instructions
  -fno-strict-aliasing                   LDS staging buffers are written and
                                         read through different types
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkvc.so")
SOURCES = [os.path.join(CSRC, f)
           for f in ("kvc_host.cpp", "kvc_pipe.cpp", "kvc_compress.hip", "kvc_decode.hip",
                     "kvc_select.hip", "kvc_pipe.hip", "kvc_rotate.hip",
                     "kvc_measure.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"


def command(out=LIB, extra=()):
    return [HIPCC, "-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero", "-fno-strict-aliasing",
            "-Xclang", "-target-feature",
            "-Xclang", "-packed-fp32-ops", "-Wall", "-Wno-unused-result",
            "-I", os.path.join(ROOT, "include"), *extra, *SOURCES, "-o", out]


def build(verbose=False):
    cmd = command()
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        raise RuntimeError("libkvc build failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    print(LIB)
    sys.exit(0)
