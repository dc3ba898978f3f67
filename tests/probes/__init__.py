"""Build and load the layout probe library (test infrastructure; see layout_probe.hip)."""
import ctypes
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "layout_probe.hip")
LIB = os.path.join(HERE, "liblayoutprobe.so")
FLAGS = ["-O3", "-std=c++17", "-fPIC", "-shared", "--offload-arch=gfx950",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build():
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    r = subprocess.run([hipcc] + FLAGS + [SRC, "-o", LIB + ".tmp"], stdout=subprocess.PIPE,
                       stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("layout probe build failed:\n" + r.stdout)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def lib():
    if not os.path.exists(LIB):
        raise ImportError(f"{LIB} is not built (run __graft_entry__.build())")
    L = ctypes.CDLL(LIB)
    vp = ctypes.c_void_p
    for name, n in (("probe_mfma_bf16", 3), ("probe_mfma_f8", 3), ("probe_tr16", 3), ("probe_tr8", 3),
                    ("probe_xlane", 2), ("probe_same_lane", 6)):
        f = getattr(L, name)
        f.argtypes = [vp] * n
        f.restype = ctypes.c_int
    return L
