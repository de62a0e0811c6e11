"""Builds the HIP libraries in-tree for gfx950 with hipcc: libmoe_decode.so (the layer) and
libmoe_bench.so (the benchmark's streaming-read reference)."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmoe_decode.so")
SOURCES = ["moe_layer.hip", "moe_api.hip", "lm_head.hip"]
BENCH_LIB = os.path.join(PKG, "libmoe_bench.so")
BENCH_SOURCES = ["bench_stream.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# -packed-fp32-ops off: no compiler-formed packed fp32 arithmetic in the device code
FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _build_lib(sources, lib, verbose):
    objs = [os.path.join(CSRC, s.replace(".hip", ".o")) for s in sources]

    def cc(i):
        cmd = [HIPCC] + FLAGS + ["-c", os.path.join(CSRC, sources[i]), "-o", objs[i]]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("hipcc failed for %s:\n%s" % (sources[i], r.stderr))
        if verbose:
            print(r.stderr, file=sys.stderr)

    with ThreadPoolExecutor(len(sources)) as ex:
        list(ex.map(cc, range(len(sources))))
    tmp = lib + ".tmp%d" % os.getpid()
    r = subprocess.run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC"] + objs + ["-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, lib)
    for o in objs:
        os.remove(o)
    return lib


def build(verbose: bool = False) -> str:
    with ThreadPoolExecutor(2) as ex:
        f_bench = ex.submit(_build_lib, BENCH_SOURCES, BENCH_LIB, verbose)
        f_main = ex.submit(_build_lib, SOURCES, LIB, verbose)
        f_bench.result()
        return f_main.result()


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
