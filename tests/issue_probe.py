"""Build and load tests/issue_probe.hip (a test helper library, not libsage)."""
import ctypes
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "issue_probe.hip")
LIB = os.path.join(HERE, "libissue_probe.so")

# instructions per chain link and links per loop iteration, by op
OPS = {0: ("v_fma_f32", 8), 1: ("v_cvt_f32_i32", 8), 2: ("v_exp_f32", 8), 3: ("v_cvt_pk_fp8_f32", 8),
       4: ("v_mfma_i32_32x32x32_i8", 4), 5: ("v_mfma_scale_f32_32x32x64_f8f6f4", 4)}


def build() -> str:
    tmp = LIB + ".tmp"
    cmd = ["hipcc", "--offload-arch=gfx950", "-O3", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for issue_probe.hip:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def load():
    if not os.path.exists(LIB):
        raise RuntimeError(f"{LIB} is missing: run __graft_entry__.build() first")
    lib = ctypes.CDLL(LIB)
    vp, i32 = ctypes.c_void_p, ctypes.c_int
    lib.probe_issue.argtypes = [i32, i32, i32, i32, vp, vp, vp]
    lib.probe_issue.restype = i32
    lib.probe_pair.argtypes = [i32, i32, i32, i32, vp, vp, vp]
    lib.probe_pair.restype = i32
    return lib
