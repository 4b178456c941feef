"""The ring's bookkeeping (csrc/ring.hip) built with g++ for the CPU under AddressSanitizer
and UndefinedBehaviorSanitizer, against a host stand-in of the HIP runtime that orders
streams and events with vector clocks (tests/ring_host/). Every read of a staged line must
happen after the copy that brought its expert, and every later copy into the line after the
read; random stagings, reads and releases on two compute streams, prefetches, the staging
waves of the host ring model, and a planted build whose release covers only its own stream
and one whose release does not wait for an unwaited fill (both of which
the check must catch)."""
import os
import shutil
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST = os.path.join(ROOT, "tests", "ring_host")
RING_SRC = os.path.join(ROOT, "routed_expert_grouped_moe_amd", "csrc", "ring.hip")


def _build(tmp, name, defines=()):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    # the ring source is copied to a .cpp of its own and compiled as host code only
    src = os.path.join(tmp, "ring_host_copy.cpp")
    shutil.copyfile(RING_SRC, src)
    exe = os.path.join(tmp, name)
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-I", HOST, "-I", os.path.join(ROOT, "routed_expert_grouped_moe_amd", "csrc"),
           *[f"-D{d}" for d in defines],
           os.path.join(HOST, "ring_host_check.cpp"), src, "-o", exe]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout[-4000:]
    return exe


@pytest.fixture(scope="module")
def exes(tmp_path_factory):
    tmp = str(tmp_path_factory.mktemp("ring_host"))
    return {"real": _build(tmp, "ring_check"),
            "planted": _build(tmp, "ring_check_planted", ["MOE_PLANT_RELEASE_ONE_STREAM=1"]),
            "planted_fill": _build(tmp, "ring_check_planted_fill",
                                   ["MOE_PLANT_RELEASE_BEFORE_FILL=1"])}


def _run(exe, *args):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    return subprocess.run([exe, *args], stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                          text=True, timeout=300, env=env)


@pytest.mark.parametrize("seed", [1, 2, 3, 4])
def test_random_sequences_are_race_free(exes, seed):
    r = _run(exes["real"], "random", str(seed), "3000")
    assert r.returncode == 0, r.stdout[-3000:]
    assert "0 races" in r.stdout


def test_release_on_a_second_stream_covers_the_first_reader(exes):
    r = _run(exes["real"], "two_streams")
    assert r.returncode == 0 and "0 races" in r.stdout, r.stdout[-3000:]
    # without the cross-stream wait the later copy may overwrite the line under the first read
    p = _run(exes["planted"], "two_streams")
    assert p.returncode == 1 and "RACE copy not after an earlier read" in p.stdout, p.stdout[-3000:]


def test_planted_build_fails_random_sequences(exes):
    bad = sum(_run(exes["planted"], "random", str(s), "3000").returncode == 1 for s in (1, 2, 3))
    assert bad >= 1


def test_release_without_waiting_for_the_fill(exes):
    """A holder may release a staged line without waiting for its copy; the release then waits
    for the copy itself, so the next copy into the line cannot overtake it. A planted build
    without that wait is caught: two copies into one line left unordered."""
    for s in (1, 2, 3):
        r = _run(exes["real"], "random", str(s), "3000")
        assert r.returncode == 0, r.stdout[-3000:]
    outs = [_run(exes["planted_fill"], "random", str(s), "3000") for s in (1, 2, 3)]
    assert any(o.returncode == 1 and "copy not after the line's previous copy" in o.stdout
               for o in outs), outs[0].stdout[-3000:]


def test_model_waves_replay(exes, tmp_path):
    """Staging waves of the host ring model (boustrophedon waves of n_lines/2, next wave
    staged ahead, near-Belady eviction) replayed through the library's staging call: the same
    hits and misses, copies by kind as the model counts them, and no race."""
    from tests.ring_model import RingModel
    rng = np.random.default_rng(7)
    E, n_lines = 24, 8
    model = RingModel(n_lines)
    for _ in range(30):
        used = sorted(rng.choice(E, size=int(rng.integers(3, 20)), replace=False).tolist())
        model.chunk(0, used)
    path = str(tmp_path / "plan.txt")
    model.write_log(path, E)
    r = _run(exes["real"], "model", path)
    assert r.returncode == 0, r.stdout[-3000:]
    line = [l for l in r.stdout.splitlines() if l.startswith("model hits")][0].split()
    hits, misses = int(line[2]), int(line[4])
    copied = [int(v) for v in line[6:10]]
    assert (hits, misses) == (model.hits, model.misses)
    assert copied == model.copied and line[-1] == "0"
    assert model.copied[0] > 0 and model.copied[1] > 0


def test_model_pinned_layer_replay(exes, tmp_path):
    """A layer call of the host model with skewed routing pins the experts most chunks use
    (held through every chunk, then released) and streams the rest; replayed through the
    library's staging and release calls: the same hits and misses, and no race."""
    from tests.ring_model import RingModel
    rng = np.random.default_rng(11)
    E, n_lines = 48, 16
    hot = list(range(10))
    model = RingModel(n_lines)
    for _ in range(3):
        chunks = [sorted(set(hot) | set(rng.choice(np.arange(10, E), size=int(rng.integers(4, 20)),
                                                 replace=False).tolist()))
                  for _ in range(12)]
        pin = model.layer(0, chunks)
        assert pin, "skewed chunks pin their hot experts"
    path = str(tmp_path / "plan.txt")
    model.write_log(path, E)
    r = _run(exes["real"], "model", path)
    assert r.returncode == 0, r.stdout[-3000:]
    line = [l for l in r.stdout.splitlines() if l.startswith("model hits")][0].split()
    assert (int(line[2]), int(line[4])) == (model.hits, model.misses)
    assert [int(v) for v in line[6:10]] == model.copied and line[-1] == "0"
