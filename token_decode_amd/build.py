"""Build the HIP library (gfx950) in-tree: token_decode_amd/libpn.so.

The kernels are split over several translation units compiled in parallel
(one per GEMM weight/activation type pair, one for attention, one for the
engine and the C ABI), then linked into one shared library.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libpn.so")
ARCH = "gfx950"

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
    # packed fp32 instructions stay off in every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]

GEMM_UNITS = [  # (weight type, activation type, entry point)
    (0, 0, "launch_gemm_f32_f32"),
    (0, 1, "launch_gemm_f32_bf16"),
    (1, 0, "launch_gemm_bf16_f32"),
    (1, 1, "launch_gemm_bf16_bf16"),
    (2, 1, "launch_gemm_i8_bf16"),
    (3, 1, "launch_gemm_q8_bf16"),
    (4, 1, "launch_gemm_q4_bf16"),
]


ATTN_UNITS = [(d, kv) for d in (32, 64, 128) for kv in (0, 1, 2)]  # kv: fp32, bf16, Q4


def _units():
    units = [("pn_lib.o", "pn_lib.hip", []), ("pn_noalloc.o", "pn_noalloc.hip", [])]
    for d, kv in ATTN_UNITS:
        units.append(("attn_%d_%d.o" % (d, kv), "pn_attn.hip",
                      ["-DPN_D=%d" % d, "-DPN_KV=%d" % kv, "-DPN_NAME=launch_attn_%d_%d" % (d, kv)]))
    for wt, at, name in GEMM_UNITS:
        units.append(("gemm_%d_%d.o" % (wt, at), "pn_gemm.hip",
                      ["-DPN_WT=%d" % wt, "-DPN_AT=%d" % at, "-DPN_NAME=%s" % name]))
    return units


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    return r.returncode, out


def build(force: bool = True, verbose: bool = False, jobs: int = None) -> str:
    """Compile libpn.so with hipcc (cross-compiles without a GPU)."""
    srcs = [os.path.join(CSRC, f) for f in os.listdir(CSRC)] + [os.path.join(ROOT, "include", "pn.h")]
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= max(map(os.path.getmtime, srcs)):
        return LIB
    os.makedirs(OBJ, exist_ok=True)
    cmds = []
    for obj, src, extra in _units():
        cmds.append(["hipcc"] + FLAGS + extra + ["-c", os.path.join(CSRC, src), "-o", os.path.join(OBJ, obj)])
    jobs = jobs or min(len(cmds), os.cpu_count() or 1, 16)
    with cf.ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_run, cmds))
    for cmd, (rc, out) in zip(cmds, results):
        if verbose or rc != 0:
            sys.stderr.write(" ".join(cmd) + "\n" + out + "\n")
        if rc != 0:
            raise RuntimeError("hipcc failed: %s" % cmd[-3])
    tmp = LIB + ".tmp%d" % os.getpid()
    rc, out = _run(["hipcc", "-shared", "-fPIC", "--offload-arch=" + ARCH] +
                   [os.path.join(OBJ, u[0]) for u in _units()] + ["-o", tmp])
    if rc != 0:
        sys.stderr.write(out + "\n")
        raise RuntimeError("linking %s failed" % LIB)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
