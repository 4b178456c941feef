"""Staging ring of expert lines (pinned host bank -> HBM on a side stream): the output of a
layer whose experts stream through the ring equals the all-resident output bit for bit, the
staging bookkeeping (hits, misses, bytes) is what the plan implies, and the error paths leave
everything unchanged. Needs an MI355X."""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle.moe_oracle as orc
from tests.parity import as_f64, logit_bound, oracle_params, place, rel_err, routing_gates

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import routed_expert_grouped_moe_amd as m
    return m


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("n_lines,offload,chunk", [
    (4, "half", 64), (1, "all", 100), (2, "all", 300), (3, "odd", 37), (64, "all", 300),
])
def test_ring_equals_resident(moe, n_lines, offload, chunk):
    wl = mi.custom_workload("ring", T=300, d=128, E=32, k=4, inter=64, inter_shared=128,
                            zipf_s=1.1, seed=21)
    E = wl.shape.n_experts
    off = {"half": range(E // 2, E), "all": range(E), "odd": range(1, E, 2)}[offload]
    params, L_res = place(wl)
    x = mi.make_x(wl, device="cuda")
    ref = moe.moe_prefill_layer(L_res, x, chunk)
    ring = moe.Ring(L_res.shape, n_lines)
    _, L_ring = place(wl, offloaded=off, ring=ring, params=params)
    cs = torch.cuda.Stream()
    got = moe.moe_prefill_layer(L_ring, x, chunk, copy_stream=cs)
    torch.cuda.synchronize()
    assert torch.equal(bits(got["out"]), bits(ref["out"]))
    st = ring.stats()
    # the host model of the plan (pinned experts, waves) predicts every count exactly
    from tests.ring_model import RingModel
    cc = ref["chunk_counts"].cpu().numpy()
    offset = np.zeros(E, bool)
    offset[list(off)] = True
    model = RingModel(n_lines)
    pin = model.layer(0, [[int(e) for e in np.nonzero(row)[0] if offset[e]] for row in cc])
    print(f"[ring] {n_lines} lines, {offload}, chunk {chunk}: pinned {len(pin)}; hits "
          f"{st['hits']} misses {st['misses']} pinned uses {st['pinned_uses']}", flush=True)
    assert (st["hits"], st["misses"], st["pinned_uses"]) == (
        model.hits, model.misses, model.pinned_uses)
    # every (chunk, used offloaded expert) pair is a hit, a copy or a use of a pinned line;
    # the pinning itself is one more staging per pinned expert
    needed = int(((cc > 0) & offset[None, :]).sum())
    assert st["hits"] + st["misses"] + st["pinned_uses"] == needed + len(pin)
    assert st["bytes_h2d"] == st["misses"] * ring.line_bytes
    assert st["misses"] >= len(set(np.nonzero(cc.sum(0) * offset)[0]))
    ring.close()


def test_ring_reuses_lines_across_calls(moe):
    """A second run finds every expert still in its line when the ring holds them all."""
    wl = mi.custom_workload("reuse", T=128, d=128, E=16, k=2, inter=64, inter_shared=64, seed=2)
    params, L_res = place(wl)
    ring = moe.Ring(L_res.shape, 16)
    _, L = place(wl, offloaded=range(16), ring=ring, params=params)
    x = mi.make_x(wl, device="cuda")
    a = moe.moe_prefill_layer(L, x, 128)
    s1 = ring.stats()
    b = moe.moe_prefill_layer(L, x, 128)
    torch.cuda.synchronize()
    s2 = ring.stats()
    assert torch.equal(bits(a["out"]), bits(b["out"]))
    assert s2["misses"] == s1["misses"] and s2["hits"] - s1["hits"] == s1["misses"]
    ring.invalidate()
    moe.moe_prefill_layer(L, x, 128)
    torch.cuda.synchronize()
    assert ring.stats()["misses"] == 2 * s1["misses"]
    ring.close()


def test_ring_passes_alternate_direction(moe):
    """Chunk passes walk the offloaded experts up, then down, then up: the lines one pass leaves
    behind are the first ones the next pass asks for, and misses evict lines the pass will
    not need again first. The ring's hit and miss counts equal those of a host model of the
    same plan (tests/ring_model.py), which also shows the gain over one fixed direction; the
    output equals the all-resident layer bit for bit."""
    from tests.ring_model import RingModel
    wl = mi.custom_workload("sweep", T=600, d=64, E=24, k=4, inter=64, inter_shared=0, seed=12)
    params, L_res = place(wl)
    x = mi.make_x(wl, device="cuda")
    ref = moe.moe_prefill_layer(L_res, x, 100)
    ring = moe.Ring(L_res.shape, 8)
    _, L = place(wl, offloaded=range(24), ring=ring, params=params)
    got = moe.moe_prefill_layer(L, x, 100, copy_stream=torch.cuda.Stream())
    torch.cuda.synchronize()
    assert torch.equal(bits(got["out"]), bits(ref["out"]))
    st = ring.stats()
    model = RingModel(8)
    cc = got["chunk_counts"].cpu().numpy()
    model.layer(0, [[int(e) for e in np.nonzero(row)[0]] for row in cc])
    print(f"[ring] sweep: library hits {st['hits']} misses {st['misses']} pinned uses "
          f"{st['pinned_uses']}; model {model.hits}/{model.misses}/{model.pinned_uses}",
          flush=True)
    assert (st["hits"], st["misses"], st["pinned_uses"]) == (
        model.hits, model.misses, model.pinned_uses)
    # one fixed direction with plain LRU (the model with every pass ascending)
    lru = RingModel(8)
    for row in cc:
        lru.sweeps = 0
        lru.chunk(0, [int(e) for e in np.nonzero(row)[0]])
    assert model.misses < lru.misses
    ring.close()


def test_pinning_falls_back_when_lines_are_held(moe):
    """A layer call that cannot pin (lines held by a caller's own staging of another layer)
    streams every expert instead: the same bytes as the all-resident layer, nothing pinned.
    The held count leaves fewer free lines than the call would pin, but room for its waves."""
    from tests.ring_model import choose_pinned
    wl = mi.custom_workload("pinfb", T=1200, d=64, E=256, k=8, inter=64, inter_shared=64,
                            zipf_s=1.5, seed=13)
    params, L_res = place(wl)
    x = mi.make_x(wl, device="cuda")
    ref = moe.moe_prefill_layer(L_res, x, 100)
    torch.cuda.synchronize()
    n_lines = 16
    cc = ref["chunk_counts"].cpu().numpy()
    want = choose_pinned([[int(e) for e in np.nonzero(r)[0]] for r in cc], n_lines, 0)
    print(f"[ring] this routing pins {len(want)} of {n_lines} lines", flush=True)
    assert len(want) > n_lines // 2, "this routing is meant to pin more than half the lines"
    held = n_lines - len(want) + 1                # one line short of the pinning
    ring = moe.Ring(L_res.shape, n_lines)
    _, L = place(wl, offloaded=range(256), ring=ring, params=params, layer=0)
    place(wl, offloaded=range(256), ring=ring, params=params, layer=1)
    cs = torch.cuda.Stream()
    lines = moe.moe_stage_experts(ring, 1, list(range(held)), copy_stream=cs)
    got = moe.moe_prefill_layer(L, x, 100, copy_stream=cs)
    torch.cuda.synchronize()
    ring.release(lines)
    assert torch.equal(bits(got["out"]), bits(ref["out"]))
    st = ring.stats()
    print(f"[ring] pin wanted {len(want)} of {n_lines} lines with {held} held elsewhere: "
          f"pinned uses {st['pinned_uses']}", flush=True)
    assert st["pinned_uses"] == 0
    # and with nothing held the same call pins
    ring.reset_stats()
    got = moe.moe_prefill_layer(L, x, 100, copy_stream=cs)
    torch.cuda.synchronize()
    assert torch.equal(bits(got["out"]), bits(ref["out"]))
    assert ring.stats()["pinned_uses"] > 0
    ring.close()


def test_stage_api_direct(moe):
    """moe_stage_experts copies exactly the bank's line into the ring line it returns."""
    wl = mi.custom_workload("stage", T=8, d=64, E=8, k=2, inter=64, inter_shared=0, seed=3)
    params, L_res = place(wl)
    ring = moe.Ring(L_res.shape, 3)
    place(wl, offloaded=range(8), ring=ring, params=params)
    cs = torch.cuda.Stream()
    lines = moe.moe_stage_experts(ring, 0, [5, 2], copy_stream=cs)
    assert len(set(lines)) == 2
    ring.wait_ready(lines)
    le = moe.line_elems(L_res.shape)
    view = ring.lines.view(torch.bfloat16).view(3, le)
    torch.cuda.synchronize()
    assert torch.equal(view[lines[0]], params["lines"][5])
    assert torch.equal(view[lines[1]], params["lines"][2])
    # 3 lines, 2 held: staging two more misses fails and changes nothing
    with pytest.raises(moe.MoeError, match="MOE_ERR_RING"):
        moe.moe_stage_experts(ring, 0, [0, 1], copy_stream=cs)
    assert ring.stats()["misses"] == 2
    # a hit needs no free line
    assert moe.moe_stage_experts(ring, 0, [5], copy_stream=cs) == [lines[0]]
    ring.release(lines)
    ring.release([lines[0]])
    l3 = moe.moe_stage_experts(ring, 0, [0, 1], copy_stream=cs)
    ring.wait_ready(l3)
    torch.cuda.synchronize()
    assert torch.equal(view[l3[0]], params["lines"][0])
    assert torch.equal(view[l3[1]], params["lines"][1])
    with pytest.raises(moe.MoeError, match="MOE_ERR_INVALID"):
        moe.moe_stage_experts(ring, 0, [3, 3], copy_stream=cs)      # duplicate
    with pytest.raises(moe.MoeError, match="MOE_ERR_RING"):
        moe.moe_stage_experts(ring, 7, [1], copy_stream=cs)          # no bank for layer 7
    ring.release(l3)
    ring.close()


def test_missing_bank_is_an_error(moe):
    wl = mi.custom_workload("nobank", T=16, d=64, E=8, k=2, inter=64, inter_shared=0, seed=4)
    params, L_res = place(wl)
    x = mi.make_x(wl, device="cuda")
    ring = moe.Ring(L_res.shape, 2)
    lines = [params["lines"][e].cuda() for e in range(8)]
    lines[3] = None
    L = moe.Layer(L_res.shape, params["w_router"], None, lines, ring=ring, layer_id=4)
    with pytest.raises(moe.MoeError, match="MOE_ERR_RING"):
        moe.moe_prefill_layer(L, x, 16)
    ring.close()


def test_ring_create_unwinds_on_failure(moe):
    """A failure while creating the ring's events returns MOE_ERR_HIP and leaves nothing
    behind (checked in a child process, since the failure is injected by an environment
    variable read at creation)."""
    code = r"""
import ctypes, torch, sys
sys.path.insert(0, sys.argv[1])
import routed_expert_grouped_moe_amd as moe
sh = moe.make_shape(64, 8, 2, 64, 0)
try:
    moe.Ring(sh, 4)
    print("created")
except moe.MoeError as e:
    print("failed", e.status)
"""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    for n, want in (("3", "failed 4"), ("8", "failed 4"), ("0", "created")):
        env = dict(os.environ, MOE_TEST_FAIL_EVENT_CREATE=n)
        out = subprocess.run([sys.executable, "-c", code, root], env=env, capture_output=True,
                             text=True, timeout=120)
        assert want in out.stdout, (n, out.stdout, out.stderr[-500:])


def test_offload_16022_ring64(moe):
    """T = 16,022, every expert in a pinned bank, 64-line ring, chunk 2,048 (as specified):
    bit-identical to the all-resident batched pass, and sampled rows match the oracle. The
    resident layer at chunks 512, 4,096 and 8,192 (16-, 128- and 256-row expert tiles against
    the batched pass's 320-row ones, at the full shape) gives the batched bytes too."""
    wl = mi.WORKLOADS["offload_16022"]
    print(f"[ring] {wl.name}: T={wl.T} E={wl.shape.n_experts} lines={wl.ring_lines}", flush=True)
    params, L_res = place(wl)
    x = mi.make_x(wl, device="cuda")
    ref = moe.moe_prefill_layer(L_res, x, wl.T)
    for c in (512, 4096, 8192):
        got_c = moe.moe_prefill_layer(L_res, x, c)
        torch.cuda.synchronize()
        assert torch.equal(bits(got_c["out"]), bits(ref["out"])), c
        del got_c
    ring = moe.Ring(L_res.shape, wl.ring_lines)
    _, L = place(wl, offloaded=range(wl.shape.n_experts), ring=ring, params=params)
    got = moe.moe_prefill_layer(L, x, 2048, copy_stream=torch.cuda.Stream())
    torch.cuda.synchronize()
    assert torch.equal(bits(got["out"]), bits(ref["out"]))
    st = ring.stats()
    assert st["bytes_h2d"] == st["misses"] * ring.line_bytes and st["waves"] >= 8
    # sampled oracle rows (the layer is per token)
    rows = np.unique(np.concatenate([np.arange(0, wl.T, 499), [wl.T - 1]]))
    op = oracle_params(params, wl)
    xs = mi.to_numpy_exact(x)[rows]
    ref_logits = orc.router_logits(xs, op["w_router"], op["router_bias"])
    ids_use, _ = routing_gates(got["logits"].cpu().numpy()[rows], got["ids"].cpu().numpy()[rows],
                               got["weights"].cpu().numpy()[rows], ref_logits, wl.shape.top_k,
                               logit_bound(xs, op["w_router"], ref_logits, wl.shape.dtype))
    err = rel_err(as_f64(got["out"])[rows], orc.moe_layer(xs, op, ids=ids_use)["out"])
    print(f"[ring] sampled rel err {err:.3e}")
    assert err <= 2e-2
    ring.close()


def test_copy_categories_match_the_model(moe):
    """The ring's requested and copied bytes by kind of staging (a chunk's first wave, a wave
    staged ahead, a wave staged on demand) equal the host model's counts, and reconcile with
    the totals."""
    from tests.ring_model import RingModel
    wl = mi.custom_workload("kinds", T=600, d=64, E=24, k=4, inter=64, inter_shared=0, seed=12)
    params, L_res = place(wl)
    x = mi.make_x(wl, device="cuda")
    for n_lines in (8, 3):
        ring = moe.Ring(L_res.shape, n_lines)
        _, L = place(wl, offloaded=range(24), ring=ring, params=params)
        got = moe.moe_prefill_layer(L, x, 100, copy_stream=torch.cuda.Stream())
        torch.cuda.synchronize()
        st = ring.stats()
        model = RingModel(n_lines)
        model.layer(0, [[int(e) for e in np.nonzero(row)[0]]
                        for row in got["chunk_counts"].cpu().numpy()])
        lb = ring.line_bytes
        kinds = ["initial", "ahead", "demand", "cross_layer"]
        print(f"[ring] kinds, {n_lines} lines: copied {[st['copied_bytes'][k] // lb for k in kinds]}"
              f" model {model.copied}", flush=True)
        assert [st["copied_bytes"][k] for k in kinds] == [c * lb for c in model.copied]
        assert [st["requested_bytes"][k] for k in kinds] == [c * lb for c in model.requested]
        assert sum(st["copied_bytes"].values()) == st["bytes_h2d"]
        assert sum(st["requested_bytes"].values()) == (st["hits"] + st["misses"]) * lb
        ring.close()


def test_prefetch_stages_without_holding(moe):
    """moe_ring_prefetch copies experts of a later layer into free lines without holding them:
    the layer's own staging then finds them as hits, the bytes count as cross-layer copies, and
    the output equals the all-resident layer bit for bit."""
    wl = mi.custom_workload("prefetch", T=64, d=128, E=16, k=2, inter=64, inter_shared=64,
                            seed=6)
    params, L_res = place(wl)
    x = mi.make_x(wl, device="cuda")
    ref = moe.moe_prefill_layer(L_res, x, 64)
    torch.cuda.synchronize()
    used = [int(e) for e in np.nonzero(ref["chunk_counts"][0].cpu().numpy())[0]]
    ring = moe.Ring(L_res.shape, 16)
    _, L = place(wl, offloaded=range(16), ring=ring, params=params, layer=3)
    cs = torch.cuda.Stream()
    ring.prefetch(3, used[:4], copy_stream=cs)
    st0 = ring.stats()
    assert st0["copied_bytes"]["cross_layer"] == 4 * ring.line_bytes and st0["misses"] == 4
    lines = moe.moe_stage_experts(ring, 3, used[4:], copy_stream=cs)   # nothing left held
    ring.release(lines)
    got = moe.moe_prefill_layer(L, x, 64, copy_stream=cs)
    torch.cuda.synchronize()
    assert torch.equal(bits(got["out"]), bits(ref["out"]))
    st = ring.stats()
    assert st["hits"] - st0["hits"] == len(used)
    with pytest.raises(moe.MoeError, match="MOE_ERR_INVALID"):
        ring.prefetch(3, [1, 1], copy_stream=cs)
    ring.close()


def test_release_on_a_second_stream_covers_the_first_reader(moe):
    """A line read on stream A and released there, then found as a hit and released on stream
    B, is refilled only after A's read: the line's one release event covers both streams. A
    bounded spin on A before its read keeps A's read late."""
    wl = mi.custom_workload("rel2", T=8, d=256, E=4, k=1, inter=64, inter_shared=0, seed=5)
    params, L_res = place(wl)
    ring = moe.Ring(L_res.shape, 1)
    place(wl, offloaded=range(4), ring=ring, params=params)
    view = ring.lines.view(torch.bfloat16)
    want = params["lines"][0].float().sum()
    cs, A, B = torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    l0 = moe.moe_stage_experts(ring, 0, [0], copy_stream=cs)
    ring.wait_ready(l0, stream=A)
    with torch.cuda.stream(A):
        torch.cuda._sleep(20_000_000)
        got = view.float().sum()
    ring.release(l0, stream=A)
    l1 = moe.moe_stage_experts(ring, 0, [0], copy_stream=cs)      # a hit
    assert l1 == l0
    ring.wait_ready(l1, stream=B)
    ring.release(l1, stream=B)
    l2 = moe.moe_stage_experts(ring, 0, [1], copy_stream=cs)      # refills the line
    ring.wait_ready(l2, stream=A)
    ring.release(l2, stream=A)
    torch.cuda.synchronize()
    assert torch.equal(got, want)
    assert torch.equal(view, params["lines"][1])
    ring.close()


_SERIAL_CHILD = r"""
import sys
import numpy as np, torch
sys.path.insert(0, sys.argv[1])
import moe_inputs as mi
import routed_expert_grouped_moe_amd as moe
from tests.parity import place
wl = mi.custom_workload("ring", T=300, d=128, E=32, k=4, inter=64, inter_shared=128,
                        zipf_s=1.1, seed=21)
params, L_res = place(wl)
ring = moe.Ring(L_res.shape, 4)
_, L = place(wl, offloaded=range(32), ring=ring, params=params)
x = mi.make_x(wl, device="cuda")
out = moe.moe_prefill_layer(L, x, 64, copy_stream=torch.cuda.Stream())["out"]
torch.cuda.synchronize()
np.save(sys.argv[2], out.view(torch.int16).cpu().numpy())
ring.close()
print("saved")
"""


def test_serialized_run_equals_async(moe, tmp_path):
    """The ring layer with every kernel and copy serialised by the runtime
    (AMD_SERIALIZE_KERNEL=3, AMD_SERIALIZE_COPY=3, in a child process) gives the bytes of the
    asynchronous run."""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    outs = {}
    for mode, extra in (("async", {}), ("serial", {"AMD_SERIALIZE_KERNEL": "3",
                                                   "AMD_SERIALIZE_COPY": "3"})):
        path = str(tmp_path / f"{mode}.npy")
        env = dict(os.environ, **extra)
        print(f"[ring] {mode} child", flush=True)
        r = subprocess.run([sys.executable, "-c", _SERIAL_CHILD, root, path], env=env,
                           capture_output=True, text=True, timeout=180, cwd=root)
        assert "saved" in r.stdout, (mode, r.stdout[-1000:], r.stderr[-2000:])
        outs[mode] = np.load(path)
    assert np.array_equal(outs["async"], outs["serial"])


def test_wrong_counts_host_stay_in_bounds(moe):
    """Caller counts that sum to n*k but differ from the chunk's own plan the waves wrongly:
    the call completes (its rows are unspecified), nothing outside the caller's tensors, the
    workspace and the ring is touched, no line stays held, and the next call with the right
    counts gives the all-resident bytes."""
    wl = mi.custom_workload("badcounts", T=300, d=128, E=32, k=4, inter=64, inter_shared=128,
                            zipf_s=1.1, seed=21)
    params, L_res = place(wl)
    x = mi.make_x(wl, device="cuda")
    ref = moe.moe_prefill_layer(L_res, x, 300)
    ring = moe.Ring(L_res.shape, 8)
    _, L = place(wl, offloaded=range(32), ring=ring, params=params)
    r = moe.moe_prefill_route(L, x, 300)
    torch.cuda.synchronize()
    counts = r["chunk_counts"][0].cpu().numpy().astype(np.int64)
    bad = counts.copy()
    i = int(np.argmax(counts))
    j = int(np.argmin(np.where(counts > 0, counts, 1 << 30)))
    bad[i] -= 60
    bad[j] += 60
    assert bad.min() >= 0 and bad.sum() == counts.sum()
    ws = torch.empty(moe.moe_workspace_bytes(L.shape, 300), dtype=torch.uint8, device="cuda")
    sentinel = torch.full((4, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    out = torch.zeros_like(x)
    cs = torch.cuda.Stream()
    moe.moe_prefill_chunk(L, x, r["ids"], r["weights"], 0, 300, out, ws,
                          counts_host=bad.tolist(), copy_stream=cs)
    torch.cuda.synchronize()
    assert torch.all(sentinel == 7.0)
    lines = moe.moe_stage_experts(ring, 0, list(range(8)), copy_stream=cs)   # every line free
    ring.release(lines)
    moe.moe_prefill_chunk(L, x, r["ids"], r["weights"], 0, 300, out, ws,
                          counts_host=counts.tolist(), copy_stream=cs)
    torch.cuda.synchronize()
    assert torch.equal(bits(out), bits(ref["out"]))
    ring.close()
