"""Build libbsa.so (the C-ABI library, HIP kernels for gfx950) in-tree with hipcc."""
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libbsa.so")
SOURCES = ["attention.hip", "select.hip", "fp8.hip", "normrope.hip", "bsa_api.hip"]
PEAK_SOURCE = "peak.hip"
PEAK_LIB = os.path.join(HERE, "libbsa_peak.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fno-strict-aliasing",
    # Packed fp32 VALU ops are disabled for the device code (see the design notes).
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def build(verbose: bool = False) -> str:
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        cmd = [HIPCC] + FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                        if "packed-fp32-ops" not in l and l.strip())
        if r.returncode != 0:
            raise RuntimeError("hipcc failed for %s:\n%s" % (src, msg))
        if verbose and msg:
            print(msg, flush=True)
        return obj

    with ThreadPoolExecutor(max_workers=len(SOURCES) + 1) as ex:
        objs = list(ex.map(compile_one, SOURCES + [PEAK_SOURCE]))
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", LIB + ".tmp"] + objs[:-1]
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    # the benchmark's MFMA throughput probe: a library of its own, outside libbsa's ABI
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", PEAK_LIB + ".tmp", objs[-1]], check=True)
    os.replace(PEAK_LIB + ".tmp", PEAK_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
