"""Stage-by-stage parity of the HIP path with the fp64 oracle, element by element, at every
routed M-tile height (16, 64, 128, 256 and 320 rows) and at the full 16,022-token layer.

For one chunk call the workspace holds the expert-major member lists, h (silu(gate) * up
rounded to the storage type), the shared expert's h and the routed experts' fp32 outputs Y
(moe_workspace_offsets). Against the oracle's stages (tests/stage_checks.py derives the
bounds):
  (i)   h and h_shared: the round-to-nearest-even value of the exact h wherever the rounding
        is decided inside the fp32 bound, a neighbour of it elsewhere;
  (ii)  Y: within the fp32 matrix-core bound of W_down times the GPU's own h;
  (iii) out: the rounding of the exact combine of the GPU's own Y and weights plus the exact
        shared output of the GPU's own h_shared, wherever decided inside the chain's bound;
  (iv)  where the shared output is exactly known (no shared expert, or a zero shared down
        projection), out equals the oracle's binary32 canonical combine of the GPU's Y and
        weights, rounded once, bit for bit.
Small-integer layers (moe_inputs.make_int_layer), whose every GEMM is exact in binary32, are
compared bit for bit at every stage: logits, ids, weights, h, Y and out.
"""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle.moe_oracle as orc
from tests import stage_checks as sc
from tests.parity import oracle_params, place

pytestmark = pytest.mark.gpu

MIN_DECIDED = 0.5     # share of elements whose rounding the bounds must decide


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import routed_expert_grouped_moe_amd as m
    m.moe_abi_version()
    return m


def _f64(a, dtype):
    """Host float64 of device data: bf16 bit patterns or fp32."""
    a = a.detach().cpu()
    if a.dtype == torch.bfloat16:
        return orc.as_f64(a.view(torch.int16).numpy().view(np.uint16))
    return a.to(torch.float64).numpy()


class Chunk:
    """One moe_prefill_chunk call over rows [t0, t0 + n) and views of its workspace."""

    def __init__(self, moe, wl, params, x, t0, n, ring=None):
        self.wl, self.params, self.t0, self.n = wl, params, t0, n
        _, L = place(wl, params=params)
        self.L = L
        sh = L.shape
        T = x.shape[0]
        r = moe.moe_prefill_route(L, x, max(n, 1))
        self.route = r
        self.ws = torch.empty(moe.moe_workspace_bytes(sh, n), dtype=torch.uint8, device="cuda")
        self.out = torch.zeros_like(x)
        moe.moe_prefill_chunk(L, x, r["ids"], r["weights"], t0, n, self.out, self.ws)
        torch.cuda.synchronize()
        o = moe.moe_workspace_offsets(sh, n)
        k, E, d, I, Is = sh.top_k, sh.n_experts, sh.d, sh.inter, sh.inter_shared
        dt = x.dtype
        esz = 2 if dt == torch.bfloat16 else 4
        i32 = lambda off, cnt: self.ws[off: off + 4 * cnt].view(torch.int32).cpu().numpy()
        self.counts = i32(o["counts"], E)
        self.offsets = i32(o["offsets"], E + 1)
        self.row_tok = i32(o["row_tok"], n * k)
        self.row_slot = i32(o["row_slot"], n * k)
        self.h_dev = self.ws[o["h"]: o["h"] + esz * n * k * I].view(dt).view(n * k, I)
        self.hs_dev = (self.ws[o["h_shared"]: o["h_shared"] + esz * n * Is].view(dt).view(n, Is)
                       if Is else None)
        self.y_dev = self.ws[o["y"]: o["y"] + 4 * n * k * d].view(torch.float32).view(n * k, d)
        self.x = x
        self.k, self.dtype = k, ("bf16" if dt == torch.bfloat16 else "f32")

    def h(self, rows):
        return _f64(self.h_dev[torch.as_tensor(rows, device="cuda").long()], None)

    def y_rows(self, slots):
        return _f64(self.y_dev[torch.as_tensor(slots, device="cuda").long()], None)

    def x_rows(self, toks):
        return _f64(self.x[torch.as_tensor(self.t0 + np.asarray(toks), device="cuda").long()], None)


def _check_routed(c, op, experts, stats):
    step = sc.STEP[c.dtype]
    for e in experts:
        a, b = int(c.offsets[e]), int(c.offsets[e + 1])
        if a == b:
            continue
        rows = np.arange(a, b)
        xr = c.x_rows(c.row_tok[rows])
        h_ref, h_bound = sc.hidden_exact_and_bound(xr, op["w_gu"][e], step)
        h_gpu = c.h(rows)
        if c.dtype == "bf16":
            n_, dec, bad = sc.rounding_check(h_gpu, h_ref, h_bound)
            stats["h"] = [stats["h"][0] + n_, stats["h"][1] + dec, stats["h"][2] + bad]
        else:
            n_, worst, bad = sc.abs_check(h_gpu, h_ref, h_bound + np.abs(h_ref) * sc.U)
            stats["h"] = [stats["h"][0] + n_, stats["h"][1] + n_, stats["h"][2] + bad]
        assert bad == 0, f"h of expert {e}: {bad} of {n_} elements outside the bound"
        y_ref, y_bound = sc.gemm_exact_and_bound(h_gpu, orc.as_f64(op["w_down"][e]), step)
        n_, worst, bad = sc.abs_check(c.y_rows(c.row_slot[rows]), y_ref, y_bound)
        stats["y_worst"] = max(stats["y_worst"], worst)
        assert bad == 0, f"Y of expert {e}: {bad} of {n_} elements outside the bound"


def _check_out(c, op, toks, stats, exact_shared=False):
    """(iii) or (iv) on chunk-local tokens toks."""
    k, step = c.k, sc.STEP[c.dtype]
    toks = np.asarray(toks)
    slots = (toks[:, None] * k + np.arange(k)[None, :]).ravel()
    y = c.y_rows(slots).reshape(len(toks), k, -1)
    w = c.route["weights"][torch.as_tensor(c.t0 + toks, device="cuda").long()].cpu().numpy()
    got = _f64(c.out[torch.as_tensor(c.t0 + toks, device="cuda").long()], None)
    if exact_shared:
        shared = None if op["w_gu_shared"] is None else np.zeros(y.shape[::2], dtype=np.float32)
        acc = orc.combine_fp32(w, y.astype(np.float32), shared).astype(np.float64)
        want = orc.bf16_rne(acc) if c.dtype == "bf16" else acc
        bad = int(np.sum(got != want))
        stats["out_exact"] = [stats["out_exact"][0] + got.size, stats["out_exact"][1] + bad]
        assert bad == 0, f"out differs from the canonical binary32 combine at {bad} elements"
        return
    s_ref, s_bound = None, None
    if op["w_gu_shared"] is not None:
        hs = _f64(c.hs_dev[torch.as_tensor(toks, device="cuda").long()], None)
        h_ref, h_bound = sc.hidden_exact_and_bound(c.x_rows(toks), op["w_gu_shared"], step)
        if c.dtype == "bf16":
            n_, dec, bad = sc.rounding_check(hs, h_ref, h_bound)
        else:
            n_, _, bad = sc.abs_check(hs, h_ref, h_bound + np.abs(h_ref) * sc.U)
            dec = n_
        stats["hs"] = [stats["hs"][0] + n_, stats["hs"][1] + dec, stats["hs"][2] + bad]
        assert bad == 0, f"h_shared: {bad} of {n_} elements outside the bound"
        s_ref, s_bound = sc.gemm_exact_and_bound(hs, orc.as_f64(op["w_down_shared"]), step)
    exact, bound = sc.chain_exact_and_bound(w, y, s_ref, s_bound)
    if c.dtype == "bf16":
        n_, dec, bad = sc.rounding_check(got, exact, bound)
    else:
        n_, _, bad = sc.abs_check(got, exact, bound + np.abs(exact) * sc.U)
        dec = n_
    stats["out"] = [stats["out"][0] + n_, stats["out"][1] + dec, stats["out"][2] + bad]
    assert bad == 0, f"out: {bad} of {n_} elements outside the bound"


def _new_stats():
    return {"h": [0, 0, 0], "hs": [0, 0, 0], "out": [0, 0, 0], "out_exact": [0, 0],
            "y_worst": 0.0}


def _report(name, stats):
    parts = []
    for key in ("h", "hs", "out"):
        n_, dec, bad = stats[key]
        if n_:
            parts.append(f"{key}: {dec}/{n_} decided")
            if key != "hs" or n_ > 1000:
                assert dec >= MIN_DECIDED * n_, (key, dec, n_)
    if stats["out_exact"][0]:
        parts.append(f"out exact: {stats['out_exact'][0]} elements")
    parts.append(f"Y worst err/bound {stats['y_worst']:.3g}")
    print(f"[stages] {name}: " + ", ".join(parts), flush=True)


SMALL = dict(d=256, E=32, k=4, inter=128, inter_shared=128)
# (t0, n) of a 2,000-token prompt for each routed tile height at E = 32, k = 4:
# n*k < 16E -> 16-row tiles; < 48E -> 64; < 128E -> 128; < 192E -> 256; < 320E -> 320
TILE_CASES = [(37, 100, 16), (11, 300, 64), (5, 600, 128), (0, 1200, 256), (0, 2000, 320)]


@pytest.mark.parametrize("t0,n,tile", TILE_CASES, ids=[f"tile{c[2]}" for c in TILE_CASES])
def test_stages_gaussian_each_tile(moe, t0, n, tile):
    wl = mi.custom_workload("stages", T=2000, zipf_s=1.1, seed=41, **SMALL)
    params = mi.make_layer(wl, device="cuda")
    x = mi.make_x(wl, device="cuda")
    print(f"[stages] gaussian E=32 k=4 d=256 t0={t0} n={n} (tile {tile})", flush=True)
    c = Chunk(moe, wl, params, x, t0, n)
    assert int(c.counts.sum()) == n * 4
    op = oracle_params(params, wl)
    stats = _new_stats()
    _check_routed(c, op, range(32), stats)
    _check_out(c, op, np.arange(n), stats)
    # the same chunk with a zero shared down projection: the shared output is exactly 0 and
    # out must be the canonical binary32 combine of the GPU's own Y and weights
    p0 = dict(params)
    p0["w_down_shared"] = torch.zeros_like(params["w_down_shared"])
    c0 = Chunk(moe, wl, p0, x, t0, n)
    op0 = oracle_params(p0, wl)
    _check_out(c0, op0, np.arange(n), stats, exact_shared=True)
    _report(f"tile {tile}", stats)


def test_stages_no_shared_expert(moe):
    """Without a shared expert the stand-alone combine kernel forms out."""
    wl = mi.custom_workload("stages_ns", T=700, d=256, E=32, k=8, inter=128, inter_shared=0,
                            zipf_s=1.1, seed=43)
    params = mi.make_layer(wl, device="cuda")
    x = mi.make_x(wl, device="cuda")
    stats = _new_stats()
    for t0, n in ((0, 700), (100, 64)):
        c = Chunk(moe, wl, params, x, t0, n)
        op = oracle_params(params, wl)
        _check_routed(c, op, range(0, 32, 3), stats)
        _check_out(c, op, np.arange(n), stats, exact_shared=True)
    _report("no shared expert", stats)


def test_stages_fp32_tiny(moe):
    wl = mi.WORKLOADS["tiny_fp32"]
    params = mi.make_layer(wl, device="cuda")
    x = mi.make_x(wl, device="cuda")
    stats = _new_stats()
    for t0, n in ((0, 40), (3, 17)):
        c = Chunk(moe, wl, params, x, t0, n)
        op = oracle_params(params, wl)
        _check_routed(c, op, range(8), stats)
        _check_out(c, op, np.arange(n), stats)
    _report("fp32 tiny", stats)


def _big_experts(c, n_pick, rng):
    """The expert with the most rows (two M-tiles when it overflows one), the fewest, and
    a seeded sample of the rest."""
    used = np.nonzero(c.counts)[0]
    pick = {int(used[np.argmax(c.counts[used])]), int(used[np.argmin(c.counts[used])])}
    pick |= set(int(e) for e in rng.choice(used, size=min(n_pick, used.size), replace=False))
    return sorted(pick)


@pytest.mark.parametrize("chunk", [16022, 2048], ids=["batched_tile320", "chunk2048_tile64"])
def test_stages_full_layer(moe, chunk):
    """The 16,022-token layer (d = 2,048, E = 512, k = 8, I = 512, I_s = 2,048) as the bench
    times it (batched: 320-row tiles) and at chunk 2,048 (64-row tiles), on sampled experts and
    tokens of the last chunk."""
    wl = mi.WORKLOADS["offload_16022"]
    params = mi.make_layer(wl, device="cuda")
    x = mi.make_x(wl, device="cuda")
    t0 = ((wl.T - 1) // chunk) * chunk
    n = wl.T - t0
    print(f"[stages] full layer T={wl.T} chunk={chunk}: rows [{t0}, {t0 + n})", flush=True)
    c = Chunk(moe, wl, params, x, t0, n)
    op = oracle_params(params, wl)
    rng = np.random.default_rng(5)
    stats = _new_stats()
    _check_routed(c, op, _big_experts(c, 6, rng), stats)
    toks = np.sort(rng.choice(n, size=min(n, 48), replace=False))
    _check_out(c, op, toks, stats)
    _report(f"full layer chunk {chunk}", stats)


# ---------------------------------------------------------------- small-integer layers

def _int_reference(op, x64, ids, k, dtype):
    """Exact stage values of a small-integer layer: h (rounded at the storage type: exact, as
    gate * up is representable), Y per (token, slot), shared S, out."""
    rne = orc.bf16_rne if dtype == "bf16" else (lambda v: v.astype(np.float32).astype(np.float64))
    T = x64.shape[0]
    y = np.zeros((T, k, x64.shape[1]))
    for e in np.unique(ids):
        t_idx, j_idx = np.nonzero(ids == e)
        h = rne(orc.expert_hidden(x64[t_idx], op["w_gu"][e])[2])
        y[t_idx, j_idx] = orc.expert_down(h, op["w_down"][e])
    s = np.zeros((T, x64.shape[1]))
    if op["w_gu_shared"] is not None:
        hs = rne(orc.expert_hidden(x64, op["w_gu_shared"])[2])
        s = orc.expert_down(hs, op["w_down_shared"])
    out = rne(y.sum(axis=1) / k + s)
    return y, s, out


INT_CASES = [("bf16", 37, 100), ("bf16", 11, 300), ("bf16", 5, 600), ("bf16", 0, 1200),
             ("bf16", 0, 2000), ("f32", 9, 300), ("f32", 0, 2000)]


@pytest.mark.parametrize("dtype,t0,n", INT_CASES,
                         ids=[f"{c[0]}_n{c[2]}" for c in INT_CASES])
def test_int_layer_bit_exact(moe, dtype, t0, n):
    """Every stage of a small-integer layer equals the exact result bit for bit."""
    wl = mi.custom_workload("int", T=2000, d=256, E=32, k=4, inter=128, inter_shared=128,
                            dtype=dtype, seed=47)
    params = mi.make_int_layer(wl, device="cuda")
    x = mi.make_int_x(wl, device="cuda")
    print(f"[stages] small-integer {dtype} t0={t0} n={n}", flush=True)
    _int_bit_exact(moe, wl, params, x, t0, n, sample=None)


def _int_bit_exact(moe, wl, params, x, t0, n, sample):
    sh = wl.shape
    k = sh.top_k
    c = Chunk(moe, wl, params, x, t0, n)
    op = oracle_params(params, wl)
    rows = np.arange(t0, t0 + n) if sample is None else t0 + sample
    x64 = _f64(x[torch.as_tensor(rows, device="cuda").long()], None)
    # routing: the planted experts, logit 1 against 0, weights exactly 1/k
    planted = np.sort(np.nonzero(x64[:, :sh.n_experts] == 1.0)[1].reshape(len(rows), k), axis=1)
    ids = c.route["ids"][torch.as_tensor(rows, device="cuda").long()].cpu().numpy()
    assert np.array_equal(ids, planted)
    lg = c.route["logits"][torch.as_tensor(rows, device="cuda").long()].cpu().numpy()
    assert np.array_equal(lg, orc.router_logits(x64, op["w_router"]))
    w = c.route["weights"][torch.as_tensor(rows, device="cuda").long()].cpu().numpy()
    assert np.all(w == np.float32(1.0 / k))
    y_ref, _, out_ref = _int_reference(op, x64, ids, k, c.dtype)
    loc = rows - t0
    slots = (loc[:, None] * k + np.arange(k)[None, :]).ravel()
    assert np.array_equal(c.y_rows(slots).reshape(y_ref.shape), y_ref), "Y"
    got = _f64(c.out[torch.as_tensor(rows, device="cuda").long()], None)
    assert np.array_equal(got, out_ref), f"out: {int(np.sum(got != out_ref))} elements differ"
    # h of every row of the sampled tokens, found through the member lists
    inv = np.empty(n * k, dtype=np.int64)
    inv[c.row_slot] = np.arange(n * k)
    r = inv[slots]
    e_of = np.searchsorted(c.offsets, r, side="right") - 1
    h_gpu = c.h(r)
    rne = orc.bf16_rne if c.dtype == "bf16" else (lambda v: v.astype(np.float32).astype(np.float64))
    for e in np.unique(e_of):
        m = e_of == e
        h_ref = rne(orc.expert_hidden(_f64(x[torch.as_tensor(t0 + c.row_tok[r[m]], device="cuda").long()], None),
                                      op["w_gu"][e])[2])
        assert np.array_equal(h_gpu[m], h_ref), f"h of expert {e}"
    if sh.inter_shared:
        hs = _f64(c.hs_dev[torch.as_tensor(loc, device="cuda").long()], None)
        assert np.array_equal(hs, rne(orc.expert_hidden(x64, op["w_gu_shared"])[2])), "h_shared"


def test_int_full_layer_bit_exact(moe):
    """A small-integer layer at the full shape (d = 2,048, E = 512, k = 8, I = 512,
    I_s = 2,048, T = 16,022) as the batched pass (320-row tiles): sampled tokens bit-exact at
    every stage; chunk 2,048 gives the same bytes."""
    wl = mi.custom_workload("int_full", T=16022, d=2048, E=512, k=8, inter=512,
                            inter_shared=2048, seed=48)
    params = mi.make_int_layer(wl, device="cuda")
    x = mi.make_int_x(wl, device="cuda")
    print("[stages] small-integer full layer T=16022 batched", flush=True)
    rng = np.random.default_rng(6)
    sample = np.sort(rng.choice(wl.T, size=64, replace=False))
    _int_bit_exact(moe, wl, params, x, 0, wl.T, sample)
    _, L = place(wl, params=params)
    a = moe.moe_prefill_layer(L, x, wl.T)["out"].clone()
    b = moe.moe_prefill_layer(L, x, 2048)["out"]
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
