"""Builds the HIP library liblatentmoe.so for gfx950 with hipcc (in-tree).

    python -m sparse_moe_layer_logits_amd.build
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "_lib")
LIB = os.path.join(OUT_DIR, "liblatentmoe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["latentmoe.hip", "route.hip", "gemm_stream.hip", "gemm_big.hip", "gemm_mid.hip", "misc.hip",
           "ssm_replay.hip"]
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
    # no packed fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("command failed: %s\n%s" % (" ".join(cmd), out))
    return out


def build(verbose: bool = False, out_dir: str = OUT_DIR) -> str:
    """Compile every source and link liblatentmoe.so into out_dir."""
    os.makedirs(out_dir, exist_ok=True)
    lib = os.path.join(out_dir, "liblatentmoe.so")
    objs = [os.path.join(out_dir, s.replace(".hip", ".o")) for s in SOURCES]

    def one(i):
        return _run([HIPCC, *FLAGS, "-c", os.path.join(CSRC, SOURCES[i]), "-o", objs[i]])

    with ThreadPoolExecutor(len(SOURCES)) as ex:
        for out in ex.map(one, range(len(SOURCES))):
            if verbose and out.strip():
                print(out)
    tmp = lib + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, lib)
    for o in objs:
        os.remove(o)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
