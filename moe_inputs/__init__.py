"""Seeded synthetic inputs for one routed mixture-of-experts layer (and a stack of them).

This module draws tensors and nothing else: activations, router weights, the router's
popularity bias and the expert weights, with the shapes and value distributions of the
workloads below. It holds no step of the layer's computation. Both the HIP path and the
fp64 oracle are fed from what it returns, so the two see identical bytes.

Value recipe (all draws fp32, then rounded to nearest-even bf16 for the bf16 workloads):
  * activations x ~ N(0, 1);
  * every expert matrix ~ N(0, 1) / sqrt(its input dimension): gate/up rows / sqrt(d),
    down rows / sqrt(inter);
  * router weight ~ N(0, 0.02^2) (standard deviation 0.02);
  * router bias (skewed workloads only): b[e] = lam * ln p[pi(e)], with p[r] proportional
    to r^-s over ranks r = 1..E (a Zipf law) and pi a seeded permutation of expert ids, so
    popular experts are scattered over the id range. lam = ZIPF_LAMBDA was set so that at
    s = 1.5 with d = 2048, E = 512, k = 8 the hottest expert takes about 10% of the
    token-slots (a check in the CPU test-suite keeps it there).

Expert weights are stored as "expert lines": one contiguous block per expert holding the
gate/up matrix [2*inter, d] (gate rows first, then up rows) followed by the down matrix
[d, inter]. The same layout serves resident weights in HBM, a pinned host bank and the
device staging ring, so staging one expert is one contiguous copy.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Optional

import numpy as np
import torch

ZIPF_LAMBDA = 0.44
ROUTER_STD = 0.02

# tensor ids used to derive independent per-tensor seeds
_T_X, _T_ROUTER, _T_BIAS, _T_LINES, _T_SHARED_GU, _T_SHARED_DN = range(6)


@dataclasses.dataclass(frozen=True)
class LayerShape:
    d: int
    n_experts: int
    top_k: int
    inter: int
    inter_shared: int
    dtype: str  # "bf16" or "f32"

    @property
    def gu_elems(self) -> int:
        return 2 * self.inter * self.d

    @property
    def line_elems(self) -> int:
        return 3 * self.inter * self.d

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    shape: LayerShape
    chunks: tuple          # chunk sizes this workload is run at (T itself = the batched pass)
    zipf_s: Optional[float]
    n_layers: int = 1
    n_offloaded: int = 0   # experts with id >= E - n_offloaded live in a pinned host bank
    ring_lines: int = 0
    rmsnorm_eps: Optional[float] = None
    seed: int = 0


_BIG = LayerShape(d=2048, n_experts=512, top_k=8, inter=512, inter_shared=2048, dtype="bf16")

WORKLOADS = {
    # tiny fp32 layer, one chunk
    "tiny_fp32": Workload("tiny_fp32", T=40,
                          shape=LayerShape(d=64, n_experts=8, top_k=2, inter=128,
                                           inter_shared=128, dtype="f32"),
                          chunks=(40,), zipf_s=None, seed=1000),
    # bf16 layer, all experts resident; chunk 1024 against the batched pass
    "layer_3001": Workload("layer_3001", T=3001, shape=_BIG, chunks=(1024, 3001),
                           zipf_s=None, seed=1001),
    # chunk-invariance gate with skewed popularity
    "chunk_gate_4099": Workload("chunk_gate_4099", T=4099, shape=_BIG,
                                chunks=(256, 1024, 2048, 4099), zipf_s=1.1, seed=1002),
    # 16,022 tokens; as specified every expert is offloaded to a pinned bank, 64-line ring
    "offload_16022": Workload("offload_16022", T=16022, shape=_BIG, chunks=(2048,),
                              zipf_s=None, n_offloaded=512, ring_lines=64, seed=1003),
    # 8-layer stack, RMSNorm + residual between layers, half the experts offloaded
    "stack_32700": Workload("stack_32700", T=32700, shape=_BIG, chunks=(2048,), zipf_s=1.5,
                            n_layers=8, n_offloaded=256, ring_lines=128, rmsnorm_eps=1e-6,
                            seed=1004),
}


def _subseed(seed: int, *path: int) -> int:
    h = hashlib.sha256(repr((int(seed),) + tuple(int(p) for p in path)).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(device, seed: int, *path: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_subseed(seed, *path))
    return g


def _normal(shape, std: float, g: torch.Generator, device, dtype) -> torch.Tensor:
    t = torch.empty(shape, dtype=torch.float32, device=device)
    t.normal_(0.0, 1.0, generator=g)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def zipf_bias(E: int, s: float, seed: int, layer: int, lam: float = ZIPF_LAMBDA) -> np.ndarray:
    """Router bias b[e] = lam * ln p[pi(e)], p Zipf(s) over ranks 1..E (fp32)."""
    rank = np.arange(1, E + 1, dtype=np.float64)
    p = rank ** (-s)
    p /= p.sum()
    perm = np.random.default_rng(_subseed(seed, layer, _T_BIAS)).permutation(E)
    b = np.empty(E, dtype=np.float64)
    b[perm] = lam * np.log(p)
    return b.astype(np.float32)


def make_x(wl: Workload, device="cpu", T: Optional[int] = None) -> torch.Tensor:
    """Activations [T, d] ~ N(0,1) in the workload dtype."""
    T = wl.T if T is None else T
    sh = wl.shape
    return _normal((T, sh.d), 1.0, _gen(device, wl.seed, 0, _T_X), device, sh.torch_dtype)


def make_layer(wl: Workload, layer: int = 0, device="cpu", experts_block: int = 64) -> dict:
    """One layer's parameters as torch tensors on `device`.

    Keys: w_router [E,d], router_bias [E] fp32 or None, lines [E, 3*inter*d] (expert lines),
    w_gu_shared [2*inter_s, d], w_down_shared [d, inter_s] (None when inter_s == 0).
    """
    sh = wl.shape
    E, d, I, Is = sh.n_experts, sh.d, sh.inter, sh.inter_shared
    dt = sh.torch_dtype
    out = {}
    out["w_router"] = _normal((E, d), ROUTER_STD, _gen(device, wl.seed, layer, _T_ROUTER),
                              device, dt)
    if wl.zipf_s is not None:
        out["router_bias"] = torch.from_numpy(zipf_bias(E, wl.zipf_s, wl.seed, layer)).to(device)
    else:
        out["router_bias"] = None
    lines = torch.empty((E, sh.line_elems), dtype=dt, device=device)
    gu = sh.gu_elems
    for e0 in range(0, E, experts_block):
        e1 = min(E, e0 + experts_block)
        g = _gen(device, wl.seed, layer, _T_LINES, e0)
        blk = torch.empty((e1 - e0, sh.line_elems), dtype=torch.float32, device=device)
        blk.normal_(0.0, 1.0, generator=g)
        blk[:, :gu].mul_(1.0 / np.sqrt(d))
        blk[:, gu:].mul_(1.0 / np.sqrt(I))
        lines[e0:e1].copy_(blk.to(dt))
        del blk
    out["lines"] = lines
    if Is > 0:
        out["w_gu_shared"] = _normal((2 * Is, d), 1.0 / np.sqrt(d),
                                     _gen(device, wl.seed, layer, _T_SHARED_GU), device, dt)
        out["w_down_shared"] = _normal((d, Is), 1.0 / np.sqrt(Is),
                                       _gen(device, wl.seed, layer, _T_SHARED_DN), device, dt)
    else:
        out["w_gu_shared"] = None
        out["w_down_shared"] = None
    return out


def split_lines(lines: torch.Tensor, sh: LayerShape):
    """Views of expert lines as (w_gu [E, 2I, d], w_down [E, d, I]); no copy."""
    E = lines.shape[0]
    gu = lines[:, : sh.gu_elems].reshape(E, 2 * sh.inter, sh.d)
    dn = lines[:, sh.gu_elems:].reshape(E, sh.d, sh.inter)
    return gu, dn


def to_numpy_exact(t: Optional[torch.Tensor]):
    """Host numpy copy that keeps every bit: bf16 -> uint16 bit patterns, else same dtype."""
    if t is None:
        return None
    t = t.detach().to("cpu")
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def custom_workload(name="custom", T=64, d=64, E=8, k=2, inter=64, inter_shared=64,
                    dtype="bf16", chunks=None, zipf_s=None, seed=7, n_layers=1,
                    rmsnorm_eps=None) -> Workload:
    """A small workload of arbitrary shape (tests, edge cases)."""
    return Workload(name, T=T, shape=LayerShape(d, E, k, inter, inter_shared, dtype),
                    chunks=tuple(chunks) if chunks else (T,), zipf_s=zipf_s,
                    n_layers=n_layers, rmsnorm_eps=rmsnorm_eps, seed=seed)


# ---------------------------------------------------------------- small-integer layers
#
# A layer whose every GEMM is exact in binary32, for bit-exact checks of the stages: integer
# activations and weights small enough that no product or partial sum needs more than 24
# bits. Routing is planted through the router: feature e < E of x is 1 exactly for the
# token's k planted experts (0 otherwise) and the router weight is the identity on those
# features, so the planted experts have logit 1 and every other expert logit 0 (ties among
# equal logits are then irrelevant) and each routing weight is exactly 1/k (k a power of
# two). Feature E is the constant 1; the rest are -1, 0 or 1. A gate row puts 26..29 on the
# constant feature and at most 7 entries of +-1 elsewhere, so gate lies in [19, 36], where
# silu(gate) equals gate to far below bf16 (and binary32) resolution; an up row has at most 7
# entries of +-1, so |up| <= 7 and |gate * up| <= 252 is exactly representable in bfloat16; a
# down row has at most 8 entries of +-1 over the intermediate features.

_T_INT_X, _T_INT_GU, _T_INT_DN, _T_INT_SGU, _T_INT_SDN = range(10, 15)


def int_layer_ok(wl: Workload) -> bool:
    sh = wl.shape
    return sh.d >= sh.n_experts + 17 and sh.top_k in (1, 2, 4, 8) and sh.top_k <= sh.n_experts


def make_int_x(wl: Workload, device="cpu", T: Optional[int] = None) -> torch.Tensor:
    """Small-integer activations [T, d] with the planted routing (see above)."""
    assert int_layer_ok(wl), "small-integer layers need d >= E + 17 and k in {1, 2, 4, 8}"
    T = wl.T if T is None else T
    sh = wl.shape
    E, d, k = sh.n_experts, sh.d, sh.top_k
    rng = np.random.default_rng(_subseed(wl.seed, 0, _T_INT_X))
    x = np.zeros((T, d), dtype=np.float32)
    for t0 in range(0, T, 4096):
        t1 = min(T, t0 + 4096)
        pick = np.argpartition(rng.random((t1 - t0, E)), k - 1, axis=1)[:, :k]
        np.put_along_axis(x[t0:t1, :E], pick, 1.0, axis=1)
    x[:, E] = 1.0
    x[:, E + 1:] = rng.integers(-1, 2, size=(T, d - E - 1)).astype(np.float32)
    return torch.from_numpy(x).to(device=device, dtype=sh.torch_dtype)


def _sparse_rows(rng, n_rows, width, lo, n_nz, const_col=None, const_range=None):
    """Dense [n_rows, width] float32 rows with n_nz entries of +-1 at columns >= lo (entries
    that land on the same column add up) and, optionally, a constant in const_range at
    const_col."""
    m = np.zeros((n_rows, width), dtype=np.float32)
    cols = rng.integers(lo, width, size=(n_rows, n_nz))
    vals = rng.choice(np.array([-1.0, 1.0], dtype=np.float32), size=(n_rows, n_nz))
    np.add.at(m, (np.repeat(np.arange(n_rows), n_nz), cols.ravel()), vals.ravel())
    if const_col is not None:
        m[:, const_col] = rng.integers(const_range[0], const_range[1] + 1, size=n_rows)
    return m


def make_int_layer(wl: Workload, layer: int = 0, device="cpu") -> dict:
    """A small-integer layer (keys as make_layer; router_bias None)."""
    assert int_layer_ok(wl), "small-integer layers need d >= E + 17 and k in {1, 2, 4, 8}"
    sh = wl.shape
    E, d, I, Is = sh.n_experts, sh.d, sh.inter, sh.inter_shared
    dt = sh.torch_dtype
    w_router = torch.zeros((E, d), dtype=dt)
    w_router[:, :E] = torch.eye(E, dtype=dt)
    lines = torch.empty((E, sh.line_elems), dtype=dt, device=device)
    for e in range(E):
        rng = np.random.default_rng(_subseed(wl.seed, layer, _T_INT_GU, e))
        gate = _sparse_rows(rng, I, d, E + 1, 7, E, (26, 29))
        up = _sparse_rows(rng, I, d, E + 1, 7)
        down = _sparse_rows(rng, d, I, 0, 8)
        line = np.concatenate([gate.ravel(), up.ravel(), down.ravel()])
        lines[e].copy_(torch.from_numpy(line).to(dt))
    out = {"w_router": w_router.to(device), "router_bias": None, "lines": lines}
    if Is > 0:
        rng = np.random.default_rng(_subseed(wl.seed, layer, _T_INT_SGU))
        gate = _sparse_rows(rng, Is, d, E + 1, 7, E, (26, 29))
        up = _sparse_rows(rng, Is, d, E + 1, 7)
        out["w_gu_shared"] = torch.from_numpy(np.concatenate([gate, up])).to(device=device, dtype=dt)
        rng = np.random.default_rng(_subseed(wl.seed, layer, _T_INT_SDN))
        out["w_down_shared"] = torch.from_numpy(_sparse_rows(rng, d, Is, 0, 8)).to(device=device, dtype=dt)
    else:
        out["w_gu_shared"] = None
        out["w_down_shared"] = None
    return out
