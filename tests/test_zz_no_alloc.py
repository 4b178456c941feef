"""moe_prefill_chunk_noalloc through the C ABI: the same bytes as moe_prefill_chunk with a
caller workspace, on two calls in a row (the second with fewer rows, so the library's array
still holds the first call's larger contents), at the full layer shape; sizes beyond the
array and offloaded experts are rejected before anything is enqueued; repeated calls leave
the device's free memory unchanged."""
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
    m.moe_abi_version()
    return m


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def test_noalloc_equals_workspace_call(moe):
    wl = mi.WORKLOADS["layer_3001"]         # d 2,048, E 512, k 8, I 512, I_s 2,048
    params, L = place(wl)
    x = mi.make_x(wl, device="cuda")
    sh = L.shape
    r = moe.moe_prefill_route(L, x, wl.T)
    cap = moe.moe_noalloc_workspace_bytes()
    print(f"[noalloc] library workspace {cap} bytes", flush=True)
    for t0, n in ((0, 1500), (1700, 300), (2990, 11)):
        assert moe.moe_workspace_bytes(sh, n) <= cap
        ws = torch.empty(moe.moe_workspace_bytes(sh, n), dtype=torch.uint8, device="cuda")
        want = torch.zeros_like(x)
        moe.moe_prefill_chunk(L, x, r["ids"], r["weights"], t0, n, want, ws)
        got = torch.full_like(x, 5.0)
        moe.moe_prefill_chunk_noalloc(L, x, r["ids"], r["weights"], t0, n, got)
        torch.cuda.synchronize()
        print(f"[noalloc] rows [{t0}, {t0 + n})", flush=True)
        assert torch.equal(bits(got[t0:t0 + n]), bits(want[t0:t0 + n])), (t0, n)
        assert torch.all(got[:t0] == 5.0) and torch.all(got[t0 + n:] == 5.0)
        del ws
    moe.moe_prefill_chunk_noalloc(L, x, r["ids"], r["weights"], 0, 1000, got)
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    for _ in range(3):
        moe.moe_prefill_chunk_noalloc(L, x, r["ids"], r["weights"], 0, 1000, got)
    torch.cuda.synchronize()
    assert torch.cuda.mem_get_info()[0] == free0
    # too many rows for the library's array: MOE_ERR_WORKSPACE, output untouched
    big = 1
    while moe.moe_workspace_bytes(sh, big) <= cap:
        big *= 2
    xb = mi.make_x(wl, device="cuda", T=big)
    ids = torch.zeros((big, sh.top_k), dtype=torch.int32, device="cuda")
    ids += torch.arange(sh.top_k, dtype=torch.int32, device="cuda")
    w = torch.full((big, sh.top_k), 1.0 / sh.top_k, dtype=torch.float32, device="cuda")
    ob = torch.full_like(xb, 3.0)
    with pytest.raises(moe.MoeError, match="MOE_ERR_WORKSPACE"):
        moe.moe_prefill_chunk_noalloc(L, xb, ids, w, 0, big, ob)
    torch.cuda.synchronize()
    assert torch.all(ob == 3.0)


def test_noalloc_rejects_offloaded_experts(moe):
    wl = mi.custom_workload("noalloc_ring", T=64, d=128, E=8, k=2, inter=64, inter_shared=64)
    params, L_res = place(wl)
    ring = moe.Ring(L_res.shape, 4)
    _, L = place(wl, offloaded=range(4), ring=ring, params=params)
    x = mi.make_x(wl, device="cuda")
    r = moe.moe_prefill_route(L_res, x, 64)
    out = torch.zeros_like(x)
    with pytest.raises(moe.MoeError, match="MOE_ERR_UNSUPPORTED"):
        moe.moe_prefill_chunk_noalloc(L, x, r["ids"], r["weights"], 0, 64, out)
    ring.close()


def test_noalloc_small_layer_two_calls(moe):
    """A second, smaller call on a shape with a shared expert and 64-row tiles, then one more
    large one: each equals the workspace call."""
    wl = mi.custom_workload("noalloc_small", T=700, d=256, E=32, k=4, inter=128,
                            inter_shared=256, zipf_s=1.1, seed=3)
    params, L = place(wl)
    x = mi.make_x(wl, device="cuda")
    r = moe.moe_prefill_route(L, x, wl.T)
    for t0, n in ((0, 700), (100, 37), (0, 700)):
        ws = torch.empty(moe.moe_workspace_bytes(L.shape, n), dtype=torch.uint8, device="cuda")
        want = torch.zeros_like(x)
        moe.moe_prefill_chunk(L, x, r["ids"], r["weights"], t0, n, want, ws)
        got = torch.zeros_like(x)
        moe.moe_prefill_chunk_noalloc(L, x, r["ids"], r["weights"], t0, n, got)
        torch.cuda.synchronize()
        assert torch.equal(bits(got), bits(want)), (t0, n)
