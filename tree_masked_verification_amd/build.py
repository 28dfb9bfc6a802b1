"""Build libtmv.so (HIP, gfx950) in-tree with hipcc."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libtmv.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def flags():
    return ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Wall", "-Wno-unused-function",
            # packed fp32 arithmetic stays off (hipcc -O3 would form v_pk_* from plain code)
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # the first kernel arguments arrive in SGPRs instead of through a dependent load
            "-mllvm", "-amdgpu-kernarg-preload-count=16",
            "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc")]


# per-source flags on top of flags()
EXTRA = {
    # MFMA accumulators in VGPRs: with 136 of them in AGPRs the register allocator copies the
    # wide LM-head kernel's accumulators between registers on every k-step (the other
    # kernels of the file keep theirs in VGPRs either way)
    "accept.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def build(verbose: bool = False) -> str:
    """Compile every HIP source into one shared library (always recompiles)."""
    objs = []
    procs = []
    os.makedirs(os.path.join(HERE, "_build"), exist_ok=True)
    for src in sources():
        obj = os.path.join(HERE, "_build", os.path.basename(src) + ".o")
        cmd = [HIPCC] + [f for f in flags() if f != "-shared"] + EXTRA.get(os.path.basename(src), []) + \
            ["-c", src, "-o", obj]
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        objs.append(obj)
    failed = False
    for src, p in procs:
        out = p.communicate()[0].decode(errors="replace")
        lines = [l for l in out.splitlines() if "packed-fp32-ops" not in l]
        if p.returncode != 0:
            failed = True
            sys.stderr.write("hipcc failed on %s:\n%s\n" % (src, "\n".join(lines)))
        elif verbose and lines:
            sys.stderr.write("\n".join(lines) + "\n")
    if failed:
        raise RuntimeError("libtmv build failed")
    tmp = LIB + ".tmp%d" % os.getpid()
    # -z defs: an unresolved symbol (e.g. a kernel stub that was not emitted) fails the link
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Wl,-z,defs", "-o", tmp] + objs)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
