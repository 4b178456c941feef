"""Checks on the compiled gfx950 code of the library (CPU only: hipcc cross-compiles).

* The GEMM mainloops issue their global->LDS stage loads as inline asm that sets M0 just
  before each load; the compiler treats M0 as reserved, so this checks that no other
  instruction of those kernels writes or reads M0.
* No kernel writes through the scalar data cache (scalar stores, scalar atomics, scalar
  cache write-back).
* No GEMM stage loop drains its loads in flight before reading a stage's fragments."""
import os
import re
import subprocess
import tempfile

import pytest

from routed_expert_grouped_moe_amd import build as B

CSRC = os.path.join(os.path.dirname(B.__file__), "csrc")


def _device_asm(src: str) -> str:
    try:
        hipcc = B._hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    flags = [f for f in B.HIP_FLAGS if f not in ("-fPIC",)]
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "k.s")
        subprocess.run([hipcc, *flags, "--cuda-device-only", "-S", os.path.join(CSRC, src),
                        "-o", out], check=True, capture_output=True)
        return open(out).read()


def _instructions(asm: str):
    for line in asm.splitlines():
        t = line.strip()
        if not t or t.startswith((";", ".", "//")) or t.endswith(":"):
            continue
        yield t


def test_m0_only_feeds_the_stage_loads():
    ins = list(_instructions(_device_asm("gemm.hip")))
    n_loads = 0
    for i, t in enumerate(ins):
        if "global_load_lds" in t:
            n_loads += 1
            assert ins[i - 1].startswith("s_mov_b32 m0,"), (ins[i - 1], t)
        elif re.search(r"\bm0\b", t):
            assert t.startswith("s_mov_b32 m0,") and "global_load_lds" in ins[i + 1], t
    assert n_loads > 0


@pytest.mark.parametrize("src", sorted(f for f in os.listdir(CSRC) if f.endswith(".hip")))
def test_no_scalar_cache_writes(src):
    for t in _instructions(_device_asm(src)):
        op = t.split()[0]
        assert not re.match(r"s_(store|buffer_store|scratch_store|atomic|buffer_atomic|dcache_wb)",
                            op), (src, t)


def test_stage_loops_keep_their_loads_in_flight():
    """The mainloop's own waits for stage loads all come before its barrier. A wait for every
    outstanding vector-memory load right before LDS fragment reads, with no barrier in
    between, was put there by the compiler, and it drains the loads the pipeline keeps in
    flight at every stage. That happened when a load issued before the mainloop was live into
    a stage loop the compiler shared between a launch's two tile kinds (decode-sized down
    30 -> 40 us); this guards against its return."""
    ins = list(_instructions(_device_asm("gemm.hip")))
    for i, t in enumerate(ins):
        if t.startswith("s_waitcnt") and "vmcnt(0)" in t:
            nxt = ins[i + 1:i + 4]
            drains = any(x.startswith("ds_read") for x in nxt) and \
                not any(x.startswith("s_barrier") for x in nxt[:2])
            assert not drains, (i, t, nxt)
