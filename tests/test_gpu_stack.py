"""A stack of MoE layers joined by RMSNorm (eps 1e-6, no gain) and a residual add, with half
of every layer's experts streamed through one staging ring shared by all layers.

Checks, per layer and teacher-forced (the oracle gets the GPU's own bf16 layer input, so the
routing gates apply): the layer output against the oracle, the residual add (one bf16
rounding of the exact sum), the RMSNorm against the oracle within half a bf16 ulp. End to end:
the final residual stream against the fp64 oracle stack on the same rows (tokens whose fp64
routing has a near-tie in some layer are reported, not compared). And the ring stack equals
the all-resident stack bit for bit. Needs an MI355X."""
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
    return t.view(torch.int16)


def _run_stack(moe, wl, rows, chunk):
    E = wl.shape.n_experts
    off = range(E - wl.n_offloaded, E) if wl.n_offloaded else range(0)
    sh = None
    params, L_res, L_ring = [], [], []
    ring = None
    for layer in range(wl.n_layers):
        p, Lr = place(wl, layer=layer)
        if ring is None:
            sh = Lr.shape
            ring = moe.Ring(sh, wl.ring_lines) if wl.n_offloaded else None
        params.append(p)
        L_res.append(Lr)
        if ring is not None:
            L_ring.append(place(wl, layer=layer, offloaded=off, ring=ring, params=p)[1])
    x = mi.make_x(wl, device="cuda")
    res = moe.moe_prefill_stack(L_res, x, chunk, wl.rmsnorm_eps, keep_inputs=True)
    if ring is not None:
        rr = moe.moe_prefill_stack(L_ring, x, chunk, wl.rmsnorm_eps,
                                   copy_stream=torch.cuda.Stream())
        torch.cuda.synchronize()
        assert torch.equal(bits(rr["out"]), bits(res["out"])), "ring stack != resident stack"
        print(f"[stack] ring stats {ring.stats()}", flush=True)
    torch.cuda.synchronize()

    eps = wl.rmsnorm_eps
    k = wl.shape.top_k
    ops = [oracle_params(p, wl) for p in params]
    worst = 0.0
    for l in range(wl.n_layers):
        h = mi.to_numpy_exact(res["inputs"][l])[rows]
        logits = res["logits"][l].cpu().numpy()[rows]
        ref_logits = orc.router_logits(h, ops[l]["w_router"], ops[l]["router_bias"])
        ids_use, _ = routing_gates(logits, res["ids"][l].cpu().numpy()[rows],
                                   res["weights"][l].cpu().numpy()[rows], ref_logits, k,
                                   logit_bound(h, ops[l]["w_router"], ref_logits,
                                               wl.shape.dtype))
        err = rel_err(as_f64(res["outs"][l])[rows], orc.moe_layer(h, ops[l], ids=ids_use)["out"])
        worst = max(worst, err)
        assert err <= 2e-2, (l, err)
        # residual add: exact sum rounded once to bf16
        xl, ol = res["x"][l], res["outs"][l]
        xn = res["x"][l + 1] if l + 1 < wl.n_layers else res["out"]
        want = (xl.double() + ol.double()).to(torch.bfloat16)
        assert torch.equal(bits(xn), bits(want)), l
        # RMSNorm of the layer input (layer 0 normalises x itself)
        hn = orc.rmsnorm(as_f64(xl)[rows], eps)
        assert np.all(np.abs(as_f64(res["inputs"][l])[rows] - hn) <= 2.0 ** -8 * np.abs(hn) + 1e-30)
    print(f"[stack] teacher-forced worst layer rel err {worst:.3e}")

    # end to end: the fp64 oracle stack on the same rows, untethered. The GPU rounds the
    # residual stream and every layer input to bf16, so a token whose top-k gap is below that
    # rounding may pick another expert than the fp64 trajectory; such tokens (different ids in
    # some layer) are counted, the others must match within the bf16 tolerance.
    xo = orc.as_f64(mi.to_numpy_exact(x)[rows])
    same = np.ones(len(rows), bool)
    for l in range(wl.n_layers):
        hn = orc.rmsnorm(xo, eps)
        r_o = orc.moe_layer(hn, ops[l])
        same &= np.all(r_o["ids"] == res["ids"][l].cpu().numpy()[rows], axis=1)
        xo = xo + r_o["out"]
    # Bound: each layer's bf16 output is held to 2e-2 (max-abs over RMS); a stack of L layers
    # compounds L such independent errors, so the end-to-end bound is 2e-2 * sqrt(L).
    err = rel_err(as_f64(res["out"])[rows][same], xo[same])
    bound = 2e-2 * np.sqrt(wl.n_layers)
    print(f"[stack] end-to-end rel err {err:.3e} (bound {bound:.3e}) over {same.sum()} of "
          f"{len(rows)} rows (the rest routed differently in some layer)")
    assert same.sum() >= 0.5 * len(rows)
    assert err <= bound
    if ring is not None:
        ring.close()


def test_stack_small(moe):
    wl = mi.Workload("stack_small", T=300,
                     shape=mi.LayerShape(d=128, n_experts=16, top_k=4, inter=64, inter_shared=64,
                                         dtype="bf16"),
                     chunks=(64,), zipf_s=1.5, n_layers=3, n_offloaded=8, ring_lines=6,
                     rmsnorm_eps=1e-6, seed=31)
    _run_stack(moe, wl, np.arange(wl.T), 64)


def test_stack_32700(moe):
    """8 layers, T = 32,700, chunk 2,048, Zipf(1.5) routing, experts 256..511 of every layer
    in pinned banks streamed through one 128-line ring; sampled rows against the oracle."""
    wl = mi.WORKLOADS["stack_32700"]
    print(f"[stack] {wl.name}: layers={wl.n_layers} T={wl.T} ring={wl.ring_lines}", flush=True)
    rows = np.unique(np.concatenate([np.arange(0, wl.T, 1553), [wl.T - 1]]))
    _run_stack(moe, wl, rows, 2048)
