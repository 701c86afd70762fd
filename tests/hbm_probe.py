"""Build and load tests/hbm_probe.hip (a test helper library, not libsage)."""
import ctypes
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "hbm_probe.hip")
LIB = os.path.join(HERE, "libhbm_probe.so")


def build() -> str:
    tmp = LIB + ".tmp"
    cmd = ["hipcc", "--offload-arch=gfx950", "-O3", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for hbm_probe.hip:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def load():
    if not os.path.exists(LIB):
        raise RuntimeError(f"{LIB} is missing: run __graft_entry__.build() first")
    lib = ctypes.CDLL(LIB)
    vp = ctypes.c_void_p
    lib.probe_read_rows.argtypes = [vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp]
    lib.probe_read_rows.restype = ctypes.c_int
    lib.probe_read_flat.argtypes = [vp, ctypes.c_size_t, ctypes.c_int, vp, vp]
    lib.probe_read_flat.restype = ctypes.c_int
    return lib
