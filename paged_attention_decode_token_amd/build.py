"""Build libpa.so (HIP kernels + C ABI) in-tree for gfx950 with hipcc."""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpa.so")
ARCH = "gfx950"


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libpa.so)")


def flags():
    # packed-fp32 ops are disabled on purpose: hand-written or compiler-made
    # v_pk_*_f32 forms are avoided in this code base
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-variable",
            "-Wno-unused-but-set-variable", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    bdir = os.path.join(HERE, "_build")
    os.makedirs(bdir, exist_ok=True)
    # the kernel instances are compiled in five shards (see the dispatch section
    # of pa_kernels.hip), in parallel with the host code
    kern = os.path.join(CSRC, "pa_kernels.hip")
    jobs = [(kern, os.path.join(bdir, "pa_kernels.%d.o" % i), ["-DPA_SHARD=%d" % i]) for i in range(5)]
    jobs.append((os.path.join(CSRC, "pa_kv_write.hip"), os.path.join(bdir, "pa_kv_write.o"), []))
    # the MQA-logits kernel reads every MFMA result at once: keep the results in
    # ordinary VGPRs instead of accumulator registers (no per-element copies)
    jobs.append((os.path.join(CSRC, "pa_mqa_logits.hip"), os.path.join(bdir, "pa_mqa_logits.o"),
                 ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]))
    jobs.append((os.path.join(CSRC, "pa_api.cpp"), os.path.join(bdir, "pa_api.cpp.o"), []))
    objs = [j[1] for j in jobs]

    def compile_one(job):
        src, obj, defs = job
        cmd = [hipcc, *flags(), *defs, "-x", "hip", "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        out = r.stdout + "".join(l + "\n" for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
        if r.returncode != 0:
            raise RuntimeError("compile failed: %s\n%s" % (" ".join(cmd), out))
        if verbose and out.strip():
            print(out, file=sys.stderr)

    with cf.ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        list(ex.map(compile_one, jobs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s%s" % (" ".join(cmd), r.stdout, r.stderr))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
