"""Builds the HIP library libmoe_decode.so in-tree for gfx950 with hipcc."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmoe_decode.so")
SOURCES = ["moe_layer.hip", "moe_api.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# -packed-fp32-ops off: no compiler-formed packed fp32 arithmetic in the device code
FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose: bool = False) -> str:
    objs = [os.path.join(CSRC, s.replace(".hip", ".o")) for s in SOURCES]

    def cc(i):
        cmd = [HIPCC] + FLAGS + ["-c", os.path.join(CSRC, SOURCES[i]), "-o", objs[i]]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("hipcc failed for %s:\n%s" % (SOURCES[i], r.stderr))
        if verbose:
            print(r.stderr, file=sys.stderr)

    with ThreadPoolExecutor(len(SOURCES)) as ex:
        list(ex.map(cc, range(len(SOURCES))))
    tmp = LIB + ".tmp%d" % os.getpid()
    r = subprocess.run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC"] + objs + ["-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    for o in objs:
        os.remove(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
