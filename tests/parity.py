"""Helpers for GPU-vs-oracle parity: placing seeded inputs on the device, widening them for
the oracle, the error metric and the routing gates. Test infrastructure only."""
from __future__ import annotations

import numpy as np
import torch

import moe_inputs as mi
import oracle.moe_oracle as orc

# Near-tie threshold for routing against fp64 logits: the GPU orders fp32 logits, which can
# swap two fp64 logits closer than this. The fp32 router dot products measured here deviate
# from the fp64 logits by about 1e-6 at d = 2,048 and 1.05e-5 at d = 16,384 (the rigorous
# per-element bound, logit_bound, is looser: it grows with the number of K steps).
TAU = 1e-4


def moe_shape(wl):
    import routed_expert_grouped_moe_amd as moe
    s = wl.shape
    return moe.make_shape(s.d, s.n_experts, s.top_k, s.inter, s.inter_shared, s.dtype)


def place(wl, layer=0, offloaded=(), ring=None, device="cuda", params=None):
    """(params on device, moe Layer) for one layer of a workload."""
    import routed_expert_grouped_moe_amd as moe
    if params is None:
        params = mi.make_layer(wl, layer, device=device)
    L = moe.Layer.from_params(params, moe_shape(wl), device, offloaded, ring, layer)
    return params, L


def oracle_params(params, wl):
    """numpy views for the oracle (bf16 kept as bit patterns, widened per expert)."""
    sh = wl.shape
    lines = mi.to_numpy_exact(params["lines"])
    E = lines.shape[0]
    gu = lines[:, : sh.gu_elems].reshape(E, 2 * sh.inter, sh.d)
    dn = lines[:, sh.gu_elems:].reshape(E, sh.d, sh.inter)
    return {
        "w_router": mi.to_numpy_exact(params["w_router"]),
        "router_bias": mi.to_numpy_exact(params["router_bias"]),
        "w_gu": gu, "w_down": dn,
        "w_gu_shared": mi.to_numpy_exact(params["w_gu_shared"]),
        "w_down_shared": mi.to_numpy_exact(params["w_down_shared"]),
        "top_k": sh.top_k,
    }


def as_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def rel_err(gpu: np.ndarray, ref: np.ndarray) -> float:
    """max |gpu - ref| / rms(ref) over the whole tensor."""
    rms = float(np.sqrt(np.mean(ref * ref)))
    return float(np.max(np.abs(gpu - ref))) / max(rms, 1e-300)


def logit_bound(x: np.ndarray, w_router: np.ndarray, ref_logits: np.ndarray,
                dtype: str) -> np.ndarray:
    """Per-element bound of |GPU logit - exact logit|: the matrix-core chain bound of
    x W_router^T (tests/stage_checks.py) plus the rounding of the fp32 bias add. x and
    w_router as the oracle takes them (bf16 bit patterns or fp32)."""
    from tests import stage_checks as sc
    _, delta = sc.gemm_exact_and_bound(orc.as_f64(x), orc.as_f64(w_router), sc.STEP[dtype])
    return delta + 2.0 * sc.U * (np.abs(ref_logits) + delta)


def routing_gates(gpu_logits: np.ndarray, gpu_ids: np.ndarray, gpu_w: np.ndarray,
                  ref_logits: np.ndarray, k: int, bound: np.ndarray, tau: float = TAU):
    """The routing checks. Returns (ids the oracle should use, number of near-tie tokens).

    (i)  the oracle's top-k applied to the GPU's own fp32 logits gives the GPU's ids exactly,
         and the oracle's weights on those logits match the GPU's to fp32 rounding;
    (ii) the GPU's logits lie within `bound` (logit_bound, per element) of the fp64 ones;
    (iii) against fp64 logits, ids agree on every token whose fp64 gap between the k-th and
         (k+1)-th logit exceeds tau; on the others every GPU-chosen logit is within tau of
         the k-th largest, and the oracle adopts the GPU's set.
    """
    g64 = gpu_logits.astype(np.float64)
    ids_on_gpu_logits = orc.select_topk(g64, k)
    assert np.array_equal(ids_on_gpu_logits, gpu_ids), "top-k of the GPU logits differs"
    w_ref = orc.topk_weights(g64, gpu_ids)
    assert np.max(np.abs(w_ref - gpu_w)) <= 2e-6, np.max(np.abs(w_ref - gpu_w))
    dev = np.abs(g64 - ref_logits)
    assert np.all(dev <= bound), f"logit off by {np.max(dev - bound):.3e} beyond its bound"
    ids_ref = orc.select_topk(ref_logits, k)
    margin = orc.topk_margin(ref_logits, k)
    diff = np.any(ids_ref != gpu_ids, axis=1)
    bad = diff & (margin > tau)
    assert not np.any(bad), f"{int(bad.sum())} tokens route differently with margin > tau"
    if np.any(diff):
        kth = -np.sort(-ref_logits, axis=1)[:, k - 1]
        chosen = np.take_along_axis(ref_logits, gpu_ids.astype(np.int64), axis=1)
        assert np.all(chosen[diff] >= kth[diff, None] - tau)
    ids_use = np.where(diff[:, None], gpu_ids, ids_ref)
    return ids_use, int(diff.sum())
