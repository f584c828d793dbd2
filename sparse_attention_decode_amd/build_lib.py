"""Build libdsa.so (the HIP kernels + C ABI) for gfx950 with hipcc."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdsa.so")
SOURCES = ["dsa_api.hip", "indexer_decode.hip", "topk.hip", "sparse_mla.hip", "cache_write.hip",
           "dcp_merge.hip", "probe.hip", "candidates.hip"]
# NaN inputs are outside the documented domain of every entry point, so min/max need not quiet
# signalling NaNs (IEEE mode off): ReLU is one v_max instead of a canonicalize plus a max.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-fno-honor-nans", "-mno-amdgpu-ieee",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-fvisibility=hidden"]


def build(verbose: bool = False, out: str = LIB, defines=()) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc, *FLAGS, *["-D" + d for d in defines], *[os.path.join(CSRC, s) for s in SOURCES],
           "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    log = "\n".join(l for l in r.stdout.splitlines()
                    if "unknown target feature" not in l and "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + log)
    if verbose and log.strip():
        print(log)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
