"""Build libmoeprefill.so in-tree with hipcc for gfx950 (MI355X).

    python -m routed_expert_grouped_moe_amd.build

Compiles every csrc/*.hip to an object in parallel, then links the shared library next to
this file. Always rebuilds (the sources are small; a stale library is worse than a rebuild).
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmoeprefill.so")
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # no packed fp32 arithmetic in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # drop the host pass's harmless note about the device-only target feature
    lines = [l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l]
    return r.returncode, "\n".join(lines)


def build(verbose: bool = False, jobs: int = 8, plants: bool = True) -> str:
    hipcc = _hipcc()
    os.makedirs(OUT_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(OUT_DIR, os.path.basename(s)[:-4] + ".o") for s in srcs]

    def compile_one(pair):
        src, obj = pair
        return src, _run([hipcc, *HIP_FLAGS, "-c", src, "-o", obj])

    failed = []
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        for src, (rc, log) in ex.map(compile_one, zip(srcs, objs)):
            if verbose and log.strip():
                print(f"[{os.path.basename(src)}]\n{log}", file=sys.stderr)
            if rc != 0:
                failed.append((src, log))
    if failed:
        msg = "\n".join(f"--- {s}\n{l}" for s, l in failed)
        raise RuntimeError(f"hipcc failed:\n{msg}")
    _link(hipcc, objs, LIB)
    if plants:
        build_plants(hipcc, srcs, objs, jobs)
    return LIB


def _link(hipcc, objs, lib):
    tmp = lib + ".tmp"
    rc, log = _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    if rc != 0:
        raise RuntimeError(f"link failed:\n{log}")
    os.replace(tmp, lib)


# Test-only builds, each with one known mistake planted (csrc/device_common.h, "planted
# mistakes"): the GPU parity tests must go red on every one of them. Only the sources that use
# the macros are compiled again; the libraries land in _build/, never next to the real one.
PLANTS = {
    "combine_desc": "MOE_PLANT_COMBINE_DESC",
    "h_trunc": "MOE_PLANT_H_TRUNC",
    "out_twice": "MOE_PLANT_OUT_TWICE",
    "korder_tall": "MOE_PLANT_KORDER_TALL",
}
_PLANTED_SOURCES = ("gemm.hip", "combine.hip")


def plant_lib(name: str) -> str:
    return os.path.join(OUT_DIR, f"libmoeprefill_plant_{name}.so")


def build_plants(hipcc, srcs, objs, jobs):
    jobs_list = []
    for name, macro in PLANTS.items():
        d = os.path.join(OUT_DIR, f"plant_{name}")
        os.makedirs(d, exist_ok=True)
        for src in srcs:
            if os.path.basename(src) in _PLANTED_SOURCES:
                jobs_list.append((name, macro, src, os.path.join(d, os.path.basename(src)[:-4] + ".o")))

    def compile_one(job):
        name, macro, src, obj = job
        return job, _run([hipcc, *HIP_FLAGS, f"-D{macro}=1", "-c", src, "-o", obj])

    failed = []
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        for job, (rc, log) in ex.map(compile_one, jobs_list):
            if rc != 0:
                failed.append((job, log))
    if failed:
        msg = "\n".join(f"--- {j[0]} {j[2]}\n{l}" for j, l in failed)
        raise RuntimeError(f"hipcc failed (planted builds):\n{msg}")
    for name in PLANTS:
        d = os.path.join(OUT_DIR, f"plant_{name}")
        pobjs = [os.path.join(d, os.path.basename(o)) if os.path.basename(o)[:-2] + ".hip"
                 in _PLANTED_SOURCES else o for o in objs]
        _link(hipcc, pobjs, plant_lib(name))


if __name__ == "__main__":
    print(build(verbose=True))
