"""Build libattn.so in-tree with hipcc for gfx950.

    python -m streaming_online_softmax_amd.build      (or __graft_entry__.build())

Every translation unit is compiled separately (in parallel) and linked into
streaming_online_softmax_amd/libattn.so.  Device code is built with packed-FP32 instructions
disabled (-packed-fp32-ops): the compiler otherwise forms v_pk_{add,mul,fma}_f32 by itself.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libattn.so")
SOURCES = ["api.cpp", "attn_fwd.hip", "attn_fwd_d256.hip", "attn_decode.hip", "attn_combine.hip", "softmax_rows.hip",
           "convert.hip", "mask_pack.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# attn_fwd*.hip: keep matrix-instruction accumulators in the VGPR form.  The D = 256 kernels need
# more than 256 registers per lane; left to itself the compiler moved their values between the
# VGPR and AGPR files about ten times per matrix instruction (measured 15% slower).  Kernels
# that fit in VGPRs are unaffected.  The D = 256 instantiations (their own translation unit) are
# also scheduled with the iterative ILP strategy: +7% (causal) and +11% (masked) measured at
# B1 H16 N16384 D256; the D <= 128 kernels measured the same under every strategy.
EXTRA = {"attn_fwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "attn_fwd_d256.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-mllvm", "-amdgpu-sched-strategy=iterative-ilp"]}


def _compile(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [HIPCC] + FLAGS + EXTRA.get(src, []) + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the packed-fp32 target feature and says so; that is harmless
    msg = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msg}")
    if msg.strip():
        print(msg, file=sys.stderr)
    return obj


def build(verbose=True):
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    # -z defs: an unresolved symbol (e.g. a kernel launch stub the host pass did not emit)
    # fails the build instead of the first dlopen
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,-z,defs", "-o", tmp] + objs
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
