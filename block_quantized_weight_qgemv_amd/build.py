"""Build libqgemv.so in-tree: the HIP kernels + C ABI (hipcc, gfx950) and the
host pack module (g++, no floating-point contraction).

    python block_quantized_weight_qgemv_amd/build.py

(run as a script: importing the package would load the library being built)
"""

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libqgemv.so")

ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
ARCH = "gfx950"

HIP_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
    # no packed fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in ordinary vector registers: left to itself the compiler
    # put the GEMM's in accumulation registers and read every result back
    # with one v_accvgpr_read per element (a quarter of the GEMM's VALU work)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    # the only atomics are one lane's LDS tile-counter increments: the
    # compiler's wave-scan rewrite of them (exec popcounts and lane offsets)
    # is work for nothing
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-I" + INCLUDE, "-I" + CSRC,
]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-ffp-contract=off",
              "-I" + INCLUDE, "-I" + os.path.join(ROCM, "include"), "-D__HIP_PLATFORM_AMD__"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        sys.stderr.write(out + "\n")
        raise RuntimeError("build step failed: %s" % " ".join(cmd))
    return out


HIP_SOURCES = ["qgemv_api.hip", "qgemv_fp4.hip", "qgemv_affine_u4.hip", "qgemv_affine_u8.hip", "qgemv_fp8.hip",
               "qgemv_q4k.hip", "qgemm.hip", "qgemv_q8.hip"]


def build(verbose=False):
    """Compile every source (in parallel: each format's kernel instances are a
    file of their own) and link libqgemv.so next to this file."""
    with tempfile.TemporaryDirectory(prefix="qgemv_build_") as tmp:
        jobs = []
        for src in HIP_SOURCES:
            obj = os.path.join(tmp, os.path.splitext(src)[0] + ".o")
            jobs.append((obj, [HIPCC] + HIP_FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]))
        pack_o = os.path.join(tmp, "pack.o")
        jobs.append((pack_o, ["g++"] + HOST_FLAGS + ["-c", os.path.join(CSRC, "pack.cpp"), "-o", pack_o]))
        procs = [(cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
                 for _, cmd in jobs]
        out, failed = "", []
        for cmd, pr in procs:
            text = pr.communicate()[0]
            text = "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l)
            out += text
            if pr.returncode != 0:
                sys.stderr.write(text + "\n")
                failed.append(" ".join(cmd))
        if failed:
            raise RuntimeError("build step failed: %s" % failed[0])
        tmp_lib = os.path.join(tmp, "libqgemv.so")
        out += _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC"] + [o for o, _ in jobs] +
                    ["-o", tmp_lib, "-lpthread"])
        shutil.move(tmp_lib, LIB)
    if verbose and out.strip():
        print(out)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
