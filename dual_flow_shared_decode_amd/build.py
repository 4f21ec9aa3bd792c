"""Builds libdfa.so in-tree for gfx950 with hipcc.

    python -m dual_flow_shared_decode_amd.build

Every HIP/C++ source under csrc/ is compiled to an object in csrc/../_build
(in parallel) and linked into dual_flow_shared_decode_amd/libdfa.so.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libdfa.so")
SOURCES = ["abi.cpp", "attn_bf16.hip", "attn_f32.hip", "combine.hip", "debug.hip", "gemv.hip", "measure.hip", "mixture.hip", "moe.hip", "noalloc.hip", "norm.hip", "prefill.hip"]
ARCH = os.environ.get("DFA_OFFLOAD_ARCH", "gfx950")
# Packed fp32 VALU ops are disabled: the compiler would otherwise form them from
# plain float code. MFMA accumulators are kept in ordinary VGPRs: the kernels
# rescale and reduce them with vector ALU code, which would otherwise copy
# them out of and back into the accumulation registers on every chunk.
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-mfma-vgpr-form=1",
         "-fvisibility=hidden", "-Wall", "-Wno-unused-function"]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the ROCm toolchain is required to build libdfa")
    return path


def _run(cmd):
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the packed-fp32 feature and says so; that is harmless
    out = "\n".join(l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()

    def compile_one(src):
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        out = _run([cc, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        if verbose and out.strip():
            print(out)
        return obj

    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    _run([cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
