"""The fused routed launch (MOE_OPT_FUSED_GU_DOWN): each 64-row M-tile runs its gate/up and
down GEMMs in one workgroup with h kept in LDS. Its Y and the layer's output must equal, bit for
bit, those of the separate gate/up and down launches (themselves checked against the oracle
stage by stage in test_gpu_stages.py), at ragged expert sizes, a partial last N-chunk, with and
without a shared expert, through the ring, and at the full 16,022-token layer; chunks it does
not cover (other tile heights, fp32, I not a multiple of 128) must run the separate launches.
The library's own launch timings show which kernels ran."""
import pytest
import torch

import moe_inputs as mi
from tests.parity import place

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import routed_expert_grouped_moe_amd as m
    m.moe_set_option("fused_gu_down", 0)
    yield m
    m.moe_set_option("fused_gu_down", 0)


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _layer(moe, L, x, chunk, fused, cs=None):
    """(out, {stage: launches}) of one layer call with the option set as given."""
    moe.moe_set_option("fused_gu_down", 1 if fused else 0)
    try:
        moe.moe_profile_read(reset=True)
        moe.moe_profile_enable(True)
        r = moe.moe_prefill_layer(L, x, chunk, copy_stream=cs)
        torch.cuda.synchronize()
        moe.moe_profile_enable(False)
        prof = moe.moe_profile_read(reset=True)
    finally:
        moe.moe_set_option("fused_gu_down", 0)
        moe.moe_profile_enable(False)
    return r["out"].clone(), {k: v[1] for k, v in prof.items()}


def _y_of_chunk(moe, L, x, chunk, t0, n, fused):
    """Y (fp32 [n*k, d]) of one moe_prefill_chunk call over rows [t0, t0 + n)."""
    sh = L.shape
    moe.moe_set_option("fused_gu_down", 1 if fused else 0)
    try:
        r = moe.moe_prefill_route(L, x, chunk)
        ws = torch.zeros(moe.moe_workspace_bytes(sh, n), dtype=torch.uint8, device="cuda")
        out = torch.zeros_like(x)
        moe.moe_prefill_chunk(L, x, r["ids"], r["weights"], t0, n, out, ws)
        torch.cuda.synchronize()
    finally:
        moe.moe_set_option("fused_gu_down", 0)
    o = moe.moe_workspace_offsets(sh, n)
    return ws[o["y"]: o["y"] + 4 * n * sh.top_k * sh.d].view(torch.int32).clone()


# (T, chunk, d, E, k, I, I_s, zipf): every chunk's experts average 16 to 48 rows, so the routed
# tiles are 64 rows tall; Zipf routing gives experts of several M-tiles and nearly empty ones
FUSED_CASES = [
    (300, 300, 256, 32, 4, 128, 256, 1.1),      # shared expert, ragged experts
    (257, 257, 320, 32, 4, 256, 0, 1.2),        # no shared expert; last N-chunk 64 columns
    (400, 200, 512, 64, 8, 512, 128, None),     # I = 512: h fills its 64 KB of LDS; two chunks
]


@pytest.mark.parametrize("T,chunk,d,E,k,I,Is,zipf", FUSED_CASES)
def test_fused_equals_separate(moe, T, chunk, d, E, k, I, Is, zipf):
    wl = mi.custom_workload("fused", T=T, d=d, E=E, k=k, inter=I, inter_shared=Is,
                            zipf_s=zipf, seed=31)
    print(f"[fused] T={T} chunk={chunk} d={d} E={E} k={k} I={I} Is={Is}", flush=True)
    _, L = place(wl)
    x = mi.make_x(wl, device="cuda")
    ref, p0 = _layer(moe, L, x, chunk, False)
    got, p1 = _layer(moe, L, x, chunk, True)
    assert p0["gu_down_fused"] == 0 and p0["gu_routed"] + p0["gu_mixed"] > 0
    assert p1["gu_down_fused"] > 0 and p1["gu_routed"] == 0 and p1["gu_mixed"] == 0
    assert p1["down_routed"] == 0
    assert torch.equal(bits(got), bits(ref))
    n = min(chunk, T)
    assert torch.equal(_y_of_chunk(moe, L, x, chunk, 0, n, True),
                       _y_of_chunk(moe, L, x, chunk, 0, n, False))


def test_fused_through_the_ring(moe):
    wl = mi.custom_workload("fused_ring", T=300, d=256, E=32, k=4, inter=128, inter_shared=256,
                            zipf_s=1.1, seed=32)
    params, L = place(wl)
    x = mi.make_x(wl, device="cuda")
    ref, _ = _layer(moe, L, x, 300, False)
    ring = moe.Ring(L.shape, 8)
    _, Lr = place(wl, offloaded=range(wl.shape.n_experts), ring=ring, params=params)
    cs = torch.cuda.Stream()
    got, p = _layer(moe, Lr, x, 300, True, cs)
    ring.close()
    assert p["gu_down_fused"] > 1 and p["gu_routed"] == 0     # one launch per wave
    assert torch.equal(bits(got), bits(ref))


@pytest.mark.parametrize("case", ["tile16", "fp32", "I192"])
def test_fused_option_leaves_other_chunks_alone(moe, case):
    kw = dict(T=300, d=256, E=32, k=4, inter=128, inter_shared=128, zipf_s=1.1, seed=33)
    chunk = 300
    if case == "tile16":
        chunk = 100                      # 12.5 rows per expert: 16-row tiles
    elif case == "fp32":
        kw["dtype"] = "f32"
    else:
        kw["inter"] = 192
    wl = mi.custom_workload("fused_off", **kw)
    _, L = place(wl)
    x = mi.make_x(wl, device="cuda")
    ref, _ = _layer(moe, L, x, chunk, False)
    got, p = _layer(moe, L, x, chunk, True)
    assert p["gu_down_fused"] == 0 and p["gu_routed"] + p["gu_mixed"] > 0
    assert torch.equal(bits(got), bits(ref))


def test_fused_full_layer_chunk2048(moe):
    """The 16,022-token layer (d = 2,048, E = 512, k = 8, I = 512, I_s = 2,048) at chunk 2,048:
    every chunk's routed tiles are 64 rows (26 to 32 rows per expert)."""
    wl = mi.WORKLOADS["offload_16022"]
    print(f"[fused] full layer T={wl.T} chunk 2048", flush=True)
    _, L = place(wl)
    x = mi.make_x(wl, device="cuda")
    ref, _ = _layer(moe, L, x, 2048, False)
    got, p = _layer(moe, L, x, 2048, True)
    assert p["gu_down_fused"] == 8 and p["gu_routed"] == 0 and p["gu_mixed"] == 0
    assert torch.equal(bits(got), bits(ref))
