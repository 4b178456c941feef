"""Pins for the fp64 oracle: checks against things other than the oracle itself (brute force
on tiny inputs, closed forms, library routines, invariants, hand-derived fixtures).

Every pin takes the oracle module as an argument so that the mutation test can run the same
pins against copies of the oracle with a planted mistake and see at least one of them fail.
"""
import itertools
import json
import os
import re

import numpy as np
from scipy.special import expit, softmax

_GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "closed_forms.json")


def _golden():
    with open(_GOLDEN) as f:
        return json.load(f)


def _close(a, b, rel=1e-12):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    scale = max(1e-300, float(np.max(np.abs(b))) if b.size else 1.0)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert a.shape == b.shape, (a.shape, b.shape)
    assert err <= rel * scale, (err, scale)


def _params(rng, d, E, k, inter, inter_s, bias=True):
    p = {
        "w_router": rng.standard_normal((E, d)) * 0.3,
        "router_bias": rng.standard_normal(E) * 0.5 if bias else None,
        "w_gu": rng.standard_normal((E, 2 * inter, d)) / np.sqrt(d),
        "w_down": rng.standard_normal((E, d, inter)) / np.sqrt(inter),
        "w_gu_shared": rng.standard_normal((2 * inter_s, d)) / np.sqrt(d) if inter_s else None,
        "w_down_shared": rng.standard_normal((d, inter_s)) / np.sqrt(inter_s) if inter_s else None,
        "top_k": k,
    }
    return p


# --- independent reference pieces (brute force; never call the oracle) -------------------

def _bf_ffn(x, w_gu, w_down):
    inter = w_gu.shape[0] // 2
    g = np.einsum("td,id->ti", x, w_gu[:inter])
    u = np.einsum("td,id->ti", x, w_gu[inter:])
    h = g * expit(g) * u
    return np.einsum("ti,di->td", h, w_down)


def _bf_select(logits_row, k):
    """Brute force: the k-subset with the largest logit sum (unique for continuous draws)."""
    E = logits_row.shape[0]
    best, best_sum = None, -np.inf
    for c in itertools.combinations(range(E), k):
        s = float(np.sum(logits_row[list(c)]))
        if s > best_sum:
            best, best_sum = c, s
    return list(best)


def _bf_layer(x, p):
    """Dense brute force: every expert on every token, then a dense weight mask."""
    T, d = x.shape
    E = p["w_router"].shape[0]
    k = p["top_k"]
    logits = np.einsum("td,ed->te", x, p["w_router"])
    if p["router_bias"] is not None:
        logits = logits + p["router_bias"]
    dense_w = np.zeros((T, E))
    for t in range(T):
        sel = _bf_select(logits[t], k)
        dense_w[t, sel] = softmax(logits[t, sel])
    Y = np.stack([_bf_ffn(x, p["w_gu"][e], p["w_down"][e]) for e in range(E)])  # [E, T, d]
    out = np.einsum("te,etd->td", dense_w, Y)
    if p["w_gu_shared"] is not None:
        out = out + _bf_ffn(x, p["w_gu_shared"], p["w_down_shared"])
    return out


# --- pins ------------------------------------------------------------------------------------

def pin_bf16_widening(o):
    g = _golden()["bf16_widening"]
    got = o.as_f64(np.array(g["bits"], dtype=np.uint16))
    for v, want in zip(got, g["values"]):
        w = float(want) if not isinstance(want, str) else float(want)
        if w == 0:
            assert v == 0 and np.signbit(v) == np.signbit(w)
        else:
            assert v == w, (v, w)
    # fp32 input keeps its value
    f = np.array([1.0000001, -3.5e-38], dtype=np.float32)
    assert np.array_equal(o.as_f64(f), f.astype(np.float64))


def pin_topk_bruteforce(o):
    rng = np.random.default_rng(11)
    for E, k in [(8, 2), (8, 3), (6, 1), (5, 5), (7, 6)]:
        logits = rng.standard_normal((40, E))
        ids = o.select_topk(logits, k)
        assert ids.shape == (40, k)
        for t in range(40):
            assert list(ids[t]) == sorted(_bf_select(logits[t], k)), (E, k, t)


def pin_topk_ties(o):
    for c in _golden()["topk_ties"]["cases"]:
        row = np.array([[float(v) for v in c["logits"]]])
        assert list(o.select_topk(row, c["k"])[0]) == c["ids"], c


def pin_topk_margin(o):
    for c in _golden()["topk_margin"]["cases"]:
        row = np.array([[float(v) for v in c["logits"]]])
        m = o.topk_margin(row, c["k"])[0]
        assert m == float(c["margin"]), (c, m)


def pin_weights_closed_form(o):
    g = _golden()["topk_weights"]
    for c in g["cases"]:
        logits = np.log(np.array([c["exp_logits"]], dtype=np.float64))
        ids = o.select_topk(logits, c["k"])
        assert list(ids[0]) == c["ids"]
        _close(o.topk_weights(logits, ids)[0], c["weights"], 1e-14)
        # a common shift of every logit changes nothing
        _close(o.topk_weights(logits + 50.0, ids)[0], c["weights"], 1e-13)
    L = g["large_logits"]
    logits = np.array([L["logits"]])
    ids = o.select_topk(logits, L["k"])
    assert list(ids[0]) == L["ids"]
    _close(o.topk_weights(logits, ids)[0], L["weights"], 1e-14)


def pin_weights_subset_softmax(o):
    rng = np.random.default_rng(12)
    logits = rng.standard_normal((64, 16)) * 2.0
    ids = o.select_topk(logits, 4)
    w = o.topk_weights(logits, ids)
    _close(w.sum(axis=1), np.ones(64), 1e-14)
    for t in range(64):
        _close(w[t], softmax(logits[t, ids[t]]), 1e-13)


def pin_silu(o):
    z = np.concatenate([np.linspace(-30, 30, 1001), [0.0, -700.0, 700.0, 1e-300]])
    _close(o.silu(z), z * expit(z), 1e-14)
    assert o.silu(np.array([0.0]))[0] == 0.0
    # silu(ln 3) = ln 3 * 3/4 (sigmoid(ln 3) = 3/4)
    _close(o.silu(np.array([np.log(3.0)])), [0.75 * np.log(3.0)], 1e-15)


def pin_ffn_roles(o):
    """Gate and up are told apart: with up fixed at 1 the expert is W_down silu(W_gate x);
    with gate fixed at c it is W_down (silu(c) * W_up x)."""
    rng = np.random.default_rng(13)
    n, d, inter = 9, 6, 4
    x = rng.standard_normal((n, d))
    x[:, 0] = 1.0
    w_gate = rng.standard_normal((inter, d))
    w_up = np.zeros((inter, d))
    w_up[:, 0] = 1.0
    w_down = rng.standard_normal((d, inter))
    g = x @ w_gate.T
    _close(o.expert_ffn(x, np.vstack([w_gate, w_up]), w_down), (g * expit(g)) @ w_down.T)
    c = 0.7
    w_gate2 = np.zeros((inter, d))
    w_gate2[:, 0] = c
    w_up2 = rng.standard_normal((inter, d))
    want = (c * expit(c) * (x @ w_up2.T)) @ w_down.T
    _close(o.expert_ffn(x, np.vstack([w_gate2, w_up2]), w_down), want)


def pin_layer_bruteforce(o):
    rng = np.random.default_rng(14)
    for (T, d, E, k, inter, inter_s, bias) in [(40, 16, 8, 2, 12, 10, True),
                                              (23, 8, 6, 3, 4, 0, False),
                                              (17, 12, 5, 1, 6, 8, True)]:
        p = _params(rng, d, E, k, inter, inter_s, bias)
        x = rng.standard_normal((T, d))
        _close(o.moe_layer(x, p)["out"], _bf_layer(x, p), 1e-12)


def pin_identical_experts(o):
    """All experts equal: weights sum to one, so routing drops out."""
    rng = np.random.default_rng(15)
    T, d, E, k, inter, inter_s = 30, 10, 6, 3, 8, 6
    p = _params(rng, d, E, k, inter, inter_s)
    p["w_gu"] = np.repeat(p["w_gu"][:1], E, axis=0)
    p["w_down"] = np.repeat(p["w_down"][:1], E, axis=0)
    x = rng.standard_normal((T, d))
    want = _bf_ffn(x, p["w_gu"][0], p["w_down"][0]) + _bf_ffn(x, p["w_gu_shared"], p["w_down_shared"])
    _close(o.moe_layer(x, p)["out"], want, 1e-12)


def pin_zero_input(o):
    rng = np.random.default_rng(16)
    p = _params(rng, 8, 5, 2, 4, 4, bias=True)
    r = o.moe_layer(np.zeros((7, 8)), p)
    assert np.array_equal(r["out"], np.zeros((7, 8)))
    # logits are the bias alone
    _close(r["logits"], np.tile(p["router_bias"], (7, 1)), 0)


def pin_k_equals_E(o):
    """k = E: a dense softmax mixture of all experts."""
    rng = np.random.default_rng(17)
    T, d, E, inter, inter_s = 12, 8, 4, 6, 4
    p = _params(rng, d, E, E, inter, inter_s)
    x = rng.standard_normal((T, d))
    logits = x @ p["w_router"].T + p["router_bias"]
    sm = softmax(logits, axis=1)
    Y = np.stack([_bf_ffn(x, p["w_gu"][e], p["w_down"][e]) for e in range(E)])
    want = np.einsum("te,etd->td", sm, Y) + _bf_ffn(x, p["w_gu_shared"], p["w_down_shared"])
    r = o.moe_layer(x, p)
    assert np.array_equal(r["ids"], np.tile(np.arange(E), (T, 1)))
    _close(r["out"], want, 1e-12)


def pin_bf16_params(o):
    """bf16 bit-pattern parameters give the same layer as their exact float64 widening."""
    rng = np.random.default_rng(18)
    p = _params(rng, 16, 6, 2, 8, 8)

    def to_bits(a):
        b = a.astype(np.float32).view(np.uint32)
        return (b >> 16).astype(np.uint16)       # truncation is fine: any bf16 value will do

    def widen(bits):
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)

    pb = dict(p)
    pf = dict(p)
    for key in ("w_router", "w_gu", "w_down", "w_gu_shared", "w_down_shared"):
        pb[key] = to_bits(p[key])
        pf[key] = widen(pb[key])
    x = rng.standard_normal((9, 16))
    xb = to_bits(x)
    _close(o.moe_layer(xb, pb)["out"], _bf_layer(widen(xb), pf), 1e-12)


def pin_member_lists(o):
    rng = np.random.default_rng(19)
    for (n, E, k) in [(37, 8, 3), (5, 16, 4), (1, 4, 4), (64, 3, 1)]:
        ids = np.sort(np.stack([rng.choice(E, k, replace=False) for _ in range(n)]), axis=1)
        counts, offsets, row_tok, row_slot = o.member_lists(ids, E)
        assert np.array_equal(counts, np.bincount(ids.ravel(), minlength=E))
        assert offsets[0] == 0 and np.array_equal(np.diff(offsets), counts)
        assert sorted(row_slot.tolist()) == list(range(n * k))            # a bijection
        assert np.array_equal(row_tok, row_slot // k)
        expert_of_row = np.repeat(np.arange(E), counts)
        assert np.array_equal(ids.ravel()[row_slot], expert_of_row)       # rows sit under their expert
        for e in range(E):
            toks = row_tok[offsets[e]:offsets[e + 1]]
            assert np.all(np.diff(toks) > 0)                              # token order in an expert


def pin_chunk_counts(o):
    rng = np.random.default_rng(20)
    T, E, k = 103, 9, 3
    ids = np.sort(np.stack([rng.choice(E, k, replace=False) for _ in range(T)]), axis=1)
    for chunk in (10, 1, 7, 103, 500):
        cc = o.chunk_counts(ids, chunk, E)
        want = np.zeros(((T + chunk - 1) // chunk, E), dtype=np.int64)
        for t in range(T):                       # token loop, brute force
            for e in ids[t]:
                want[t // chunk, e] += 1
        assert np.array_equal(cc, want), chunk
        assert np.array_equal(cc.sum(axis=0), np.bincount(ids.ravel(), minlength=E))


def pin_rmsnorm(o):
    g = _golden()["rmsnorm_constant_row"]
    for c, want in g["cases"]:
        got = o.rmsnorm(np.full((1, 8), c), g["eps"])
        _close(got, np.full((1, 8), want), 1e-15)
    rng = np.random.default_rng(21)
    x = rng.standard_normal((5, 32)) * 3.0
    want = x / (np.linalg.norm(x, axis=1, keepdims=True) / np.sqrt(32))
    _close(o.rmsnorm(x, 0.0), want, 1e-14)
    _close(o.rmsnorm(5.0 * x, 0.0), o.rmsnorm(x, 0.0), 1e-14)


def pin_stack(o):
    rng = np.random.default_rng(22)
    d = 12
    x = rng.standard_normal((15, d)) * 2.0
    p1 = _params(rng, d, 6, 2, 8, 6)
    p2 = _params(rng, d, 6, 2, 8, 6)
    # composition against the brute-force layer on the hand-normalised input
    xn = x / (np.linalg.norm(x, axis=1, keepdims=True) / np.sqrt(d))
    _close(o.moe_stack(x, [p1], 0.0), x + _bf_layer(xn, p1), 1e-12)
    # zero down projections: every layer adds nothing
    pz = dict(p2)
    pz["w_down"] = np.zeros_like(p2["w_down"])
    pz["w_down_shared"] = np.zeros_like(p2["w_down_shared"])
    assert np.array_equal(o.moe_stack(x, [pz, pz], 1e-6), x)
    _close(o.moe_stack(x, [p1, pz], 1e-6), o.moe_stack(x, [p1], 1e-6), 0)
    # the layer sees a normalised input: scaling x scales only the residual part
    _close(o.moe_stack(2.0 * x, [p1], 0.0) - 2.0 * x, o.moe_stack(x, [p1], 0.0) - x, 1e-12)


def pin_chunk_invariance(o):
    """The layer is per token: any split of the rows gives the same rows back."""
    rng = np.random.default_rng(23)
    p = _params(rng, 16, 8, 3, 8, 8)
    x = rng.standard_normal((50, 16))
    full = o.moe_layer(x, p)["out"]
    for c in (7, 1, 16, 50):
        parts = np.concatenate([o.moe_layer(x[i:i + c], p)["out"] for i in range(0, 50, c)])
        _close(parts, full, 1e-13)



# --- rounding points (hand-derived fixtures, library routines) ---------------------------

_ROUNDING = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                         "rounding_points.json")


def _num(text):
    """A fixture number: a short arithmetic expression over integers and powers of two."""
    t = text.strip()
    if t in ("inf", "-inf", "-0.0"):
        return float(t)
    assert re.fullmatch(r"[0-9+\-*/(). ^]+", t), t
    return float(eval(t.replace("^", "**"), {"__builtins__": {}}, {}))


def _rounding():
    with open(_ROUNDING) as f:
        return json.load(f)


def _same(a, b):
    return (a == b and np.signbit(a) == np.signbit(b)) or (np.isnan(a) and np.isnan(b))


def pin_bf16_rne(o):
    """Hand-derived ties, spacing changes, subnormals and overflow; then torch's own
    binary32 -> bfloat16 conversion (round to nearest even) on random bit patterns and on
    exact ties (low half 0x8000)."""
    for c in _rounding()["bf16_rne"]:
        got = float(o.bf16_rne(np.array([_num(c["in"])]))[0])
        assert _same(got, _num(c["out"])), c
    import torch
    rng = np.random.default_rng(31)
    bits = rng.integers(0, 2 ** 32, size=200000, dtype=np.uint64).astype(np.uint32)
    ties = (bits[:50000] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    f = np.concatenate([bits, ties]).view(np.float32)
    f = f[np.isfinite(f)]
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).to(torch.float64).numpy()
    got = o.bf16_rne(f.astype(np.float64))
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(want))


def _libm_fmaf():
    import ctypes
    import ctypes.util
    m = ctypes.CDLL(ctypes.util.find_library("m"))
    m.fmaf.restype = ctypes.c_float
    m.fmaf.argtypes = [ctypes.c_float] * 3
    return m.fmaf


def pin_fma_f32(o):
    """Hand-derived fused cases, then the C library's fmaf (correctly rounded) on random
    triples, many of them cancelling (c close to -a*b)."""
    for c in _rounding()["fma_f32"]:
        got = float(o.fma_f32(np.float32(_num(c["a"])), np.float32(_num(c["b"])),
                              np.float32(_num(c["c"]))))
        assert _same(got, _num(c["out"])), c
    fmaf = _libm_fmaf()
    rng = np.random.default_rng(32)
    a = (rng.standard_normal(3000) * np.exp2(rng.integers(-20, 20, 3000))).astype(np.float32)
    b = (rng.standard_normal(3000) * np.exp2(rng.integers(-20, 20, 3000))).astype(np.float32)
    c = (rng.standard_normal(3000) * np.exp2(rng.integers(-40, 40, 3000))).astype(np.float32)
    c[:1500] = -(a[:1500] * b[:1500]) * (1 + rng.integers(-4, 5, 1500) * 2.0 ** -23)
    got = o.fma_f32(a, b, c)
    want = np.array([fmaf(float(x), float(y), float(z)) for x, y, z in zip(a, b, c)],
                    dtype=np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def pin_combine_fp32(o):
    """Order and fusion witnesses (hand-derived), then a slot-by-slot loop over the C
    library's fmaf in ascending slot order with the shared output added last."""
    for c in _rounding()["combine_fp32"]:
        w = np.array([[_num(v) for v in c["w"]]], dtype=np.float32)
        y = np.array([[[_num(v)] for v in c["y"]]], dtype=np.float32)
        sh = None if c["shared"] is None else np.array([[_num(c["shared"])]], dtype=np.float32)
        got = float(o.combine_fp32(w, y, sh)[0, 0])
        assert _same(got, _num(c["out"])), c
    fmaf = _libm_fmaf()
    rng = np.random.default_rng(33)
    n, k, d = 6, 5, 7
    w = rng.random((n, k)).astype(np.float32)
    y = rng.standard_normal((n, k, d)).astype(np.float32)
    sh = rng.standard_normal((n, d)).astype(np.float32)
    got = o.combine_fp32(w, y, sh)
    for t in range(n):
        for col in range(d):
            acc = 0.0
            for j in range(k):
                acc = fmaf(float(w[t, j]), float(y[t, j, col]), acc)
            want = np.float32(acc) + sh[t, col]
            assert got[t, col].view(np.uint32) == np.float32(want).view(np.uint32)


def pin_expert_stages(o):
    """gate/up/h on a hand example (h = 2 silu(1)), and the stages compose to the expert."""
    g, u, h = o.expert_hidden(np.array([[1.0, 2.0]]), np.array([[1.0, 0.0], [0.0, 1.0]]))
    assert g[0, 0] == 1.0 and u[0, 0] == 2.0
    _close(h, [[2.0 / (1.0 + np.exp(-1.0))]], 1e-15)
    rng = np.random.default_rng(34)
    x = rng.standard_normal((9, 6))
    wgu = rng.standard_normal((10, 6))
    wd = rng.standard_normal((6, 5))
    g, u, h = o.expert_hidden(x, wgu)
    _close(g, x @ wgu[:5].T, 1e-14)
    _close(u, x @ wgu[5:].T, 1e-14)
    _close(h, g * expit(g) * u, 1e-14)
    _close(o.expert_down(h, wd), np.einsum("ti,di->td", h, wd), 1e-13)
    _close(o.expert_ffn(x, wgu, wd), _bf_ffn(x, wgu, wd), 1e-13)


ALL_PINS = [v for k_, v in sorted(globals().items()) if k_.startswith("pin_")]
