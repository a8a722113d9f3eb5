"""Build the HIP library (gfx950) in-tree: token_decode_amd/libpn.so."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "pn_lib.hip")
HDRS = [os.path.join(HERE, "csrc", "pn_kernels.hpp"), os.path.join(ROOT, "include", "pn.h")]
LIB = os.path.join(HERE, "libpn.so")
ARCH = "gfx950"

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", "--offload-arch=" + ARCH,
    # packed fp32 instructions stay off in every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


def build(force: bool = True, verbose: bool = False) -> str:
    """Compile libpn.so with hipcc (cross-compiles without a GPU)."""
    if not force and os.path.exists(LIB):
        newest = max(os.path.getmtime(p) for p in [SRC] + HDRS)
        if os.path.getmtime(LIB) >= newest:
            return LIB
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["hipcc"] + FLAGS + ["-I", os.path.join(ROOT, "include"), SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        sys.stderr.write(out + "\n")
        raise RuntimeError("hipcc failed building %s" % LIB)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
