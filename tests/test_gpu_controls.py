"""Planted controls: test builds of the library, each with one known mistake (a combine in
descending expert order, h truncated instead of rounded, the routed sum rounded before the
shared output is added, a K order that depends on the M-tile height), must each fail the
parity check aimed at it. Each runs in a child process that loads the planted library in
place of the real one; the real library passes the same checks in test_gpu_stages.py and
test_gpu_parity.py."""
import os
import subprocess
import sys

import pytest
import torch

from routed_expert_grouped_moe_amd.build import PLANTS, plant_lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", sorted(PLANTS))
def test_planted_mistake_fails_its_check(name):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lib = plant_lib(name)
    assert os.path.exists(lib), f"{lib} missing: build the library (it builds the controls too)"
    print(f"[control] running {name}", flush=True)
    r = subprocess.run([sys.executable, "-u", "-m", "tests.planted_check", name, lib], cwd=ROOT,
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=240)
    print(r.stdout[-2000:], flush=True)
    assert r.returncode == 0, r.stdout[-4000:]
    assert f"CONTROL_RED {name}" in r.stdout, f"the planted mistake {name} passed its check"
