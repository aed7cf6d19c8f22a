"""Builds the HIP library libkda.so for gfx950 with hipcc, in-tree.

Each csrc/*.hip translation unit is compiled in parallel, then linked into
gated_delta_rule_gate_amd/_build/libkda.so.
"""
import concurrent.futures as cf
import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(OUT_DIR, "libkda.so")
ARCH = "gfx950"

# Packed FP32 vector ops are disabled: the compiler would otherwise form
# v_pk_* FP32 instructions from ordinary float code.
HIPCC_FLAGS = ["-O3", "-std=c++20", "-fPIC", "--offload-arch=" + ARCH,
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Wno-unused-result"]


def _hipcc():
    for cand in ("/opt/rocm/bin/hipcc", "hipcc"):
        if os.path.sep not in cand or os.path.exists(cand):
            return cand
    return "hipcc"


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _compile(src):
    obj = os.path.join(OUT_DIR, os.path.basename(src)[:-4] + ".o")
    cmd = [_hipcc()] + HIPCC_FLAGS + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, r.stdout, r.stderr))
    return obj


def build(jobs: int = 8) -> str:
    """Compiles every kernel and the host API; returns the path of libkda.so."""
    os.makedirs(OUT_DIR, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(srcs)))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [_hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH] + objs + ["-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (r.stdout, r.stderr))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
