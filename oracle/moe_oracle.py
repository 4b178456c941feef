"""fp64 CPU oracle for one routed mixture-of-experts layer with an always-on shared expert,
and for a stack of such layers joined by RMSNorm and a residual add.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or link this module:
only the test-suite, the smoke check and the benchmark's CPU-baseline leg use it. It shares
no code with the HIP path; the two meet only at the seeded inputs.

What it computes, and where that comes from
-------------------------------------------
The pages ("Flash Next EXL3: exact deep prefill", PR #1443, opening section) describe
expert-major deep-prefill chunks that use one canonical routed-expert reduction, so that
deep prefill gives the batched pass's bytes at any chunk size (the equality gate at chunk
sizes 256 / 1,024 / 2,048 in its "Completed final functional audit" section). Deep prefill
therefore reaches exactly the plain layer result, only in a fixed order, and the oracle is
that plain result written out per token, in float64:

  1. router logits  l[t, e] = sum_i x[t, i] * W_r[e, i] + b[e]
  2. top-k: the k largest logits of token t; among equal logits the lower expert id wins;
     the chosen ids are listed in ascending id order
  3. weights: softmax of l[t, :] over all E experts, renormalised over the chosen k
  4. each chosen expert e: gate = W_gate,e x, up = W_up,e x, h = silu(gate) * up,
     y_e = W_down,e h, with silu(z) = z / (1 + exp(-z)); W_gu holds the gate rows first,
     then the up rows (the pages name gate/up ("GU") and down expert kernels in the
     "Completed device checks" and numerical-audit sections of that page, no formulas)
  5. the shared expert (PR #1113, "Memory and execution split": a resident shared expert
     beside the routed ones) gives s_t the same way, with weight 1
  6. out_t = sum over chosen e in ascending id of w[t, e] * y_e, plus s_t
  7. stack: x <- x + layer(x / sqrt(mean(x^2) + eps)) (RMSNorm without gain, pre-norm)

Steps 2-7 are readings of what the pages leave open; each is listed with its reason in the
design notes. Member lists (which rows each expert processes, in token order) and per-chunk
expert counts are integer bookkeeping whose definition is unique; they are written out too.

Parity pins: every function here is checked in the CPU test-suite against brute force,
closed forms, library routines and invariants, not against itself.
"""
from __future__ import annotations

import numpy as np


# ---------------------------------------------------------------- input widening

def as_f64(a):
    """Exact float64 copy. uint16 arrays are bf16 bit patterns (upper half of an fp32)."""
    if a is None:
        return None
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


# ---------------------------------------------------------------- routing

def router_logits(x, w_router, bias=None):
    """l = x W_r^T + b, float64. x [T, d], w_router [E, d], bias [E] or None."""
    logits = as_f64(x) @ as_f64(w_router).T
    if bias is not None:
        logits = logits + as_f64(bias)[None, :]
    return logits


def select_topk(logits, k):
    """ids [T, k]: each row's k largest logits (lower id first among equal values), then
    sorted by ascending expert id."""
    logits = np.asarray(logits, dtype=np.float64)
    # a stable sort of -l keeps equal values in ascending id order
    order = np.argsort(-logits, axis=1, kind="stable")
    return np.sort(order[:, :k], axis=1)


def topk_margin(logits, k):
    """l_(k) - l_(k+1) per row: the gap between the k-th and (k+1)-th largest logit
    (+inf when k equals the number of experts)."""
    logits = np.asarray(logits, dtype=np.float64)
    E = logits.shape[1]
    if k >= E:
        return np.full(logits.shape[0], np.inf)
    srt = -np.sort(-logits, axis=1)
    return srt[:, k - 1] - srt[:, k]


def topk_weights(logits, ids):
    """Routing weights [T, k]: softmax over all experts, renormalised over the chosen ids."""
    logits = np.asarray(logits, dtype=np.float64)
    p = np.exp(logits - logits.max(axis=1, keepdims=True))
    p = p / p.sum(axis=1, keepdims=True)
    chosen = np.take_along_axis(p, np.asarray(ids), axis=1)
    return chosen / chosen.sum(axis=1, keepdims=True)


# ---------------------------------------------------------------- expert FFN

def silu(z):
    return z / (1.0 + np.exp(-z))


def expert_hidden(xr, w_gu):
    """The gate/up stage of one SwiGLU expert on rows xr [n, d] with w_gu [2I, d] (gate rows,
    then up rows): returns (gate, up, h) [n, I] float64 with h = silu(gate) * up. This is the
    gate/up ("GU") kernel's result before any rounding of h (the exact deep prefill page,
    "Flash Next EXL3: exact deep prefill", names the split into GU and down expert kernels
    in its numerical-phase audit)."""
    xr = as_f64(xr)
    w_gu = as_f64(w_gu)
    inter = w_gu.shape[0] // 2
    gate = xr @ w_gu[:inter].T
    up = xr @ w_gu[inter:].T
    return gate, up, silu(gate) * up


def expert_down(h, w_down):
    """The down stage of one expert: h [n, I] times w_down [d, I] transposed, [n, d] float64."""
    return as_f64(h) @ as_f64(w_down).T


def expert_ffn(xr, w_gu, w_down):
    """One SwiGLU expert on rows xr [n, d]: w_gu [2I, d] (gate rows, then up rows),
    w_down [d, I]. Returns [n, d] float64."""
    return expert_down(expert_hidden(xr, w_gu)[2], w_down)


# ---------------------------------------------------------------- rounding points
#
# The plain result above is what the method reaches up to rounding. The pages fix where a
# deep-prefill result may be rounded: fp32 accumulation inside the expert kernels, and one
# rounding of each routed/shared sum at the finish ("Flash Next EXL3: exact deep prefill",
# numerical-phase audit; "deep prefill (3/8)", the TP-partials item of its checklist). The
# canonical reduction order itself is a reading: each token's expert contributions are
# added in ascending expert id, the shared expert's output last. The functions below write
# those rounding points out exactly, so a GPU result can be compared with them bit for bit.

def bf16_rne(v):
    """Nearest bfloat16 value of each float64 value, ties to the even significand, returned
    as float64. bfloat16 is binary32 with 8 significant bits: a finite value with
    2^(e-1) <= |v| < 2^e is a multiple of 2^(e-8), and below 2^-126 every value is a
    multiple of 2^-133 (the subnormal spacing). Values that round to 2^128 or beyond become
    infinite; zeros keep their sign; NaN stays NaN."""
    v = np.array(v, dtype=np.float64, copy=True)
    out = v.copy()
    fin = np.isfinite(v) & (v != 0)
    if np.any(fin):
        vf = v[fin]
        _, e = np.frexp(vf)                         # vf = m * 2^e with 1/2 <= |m| < 1
        q = np.maximum(e - 8, -133)                 # exponent of the spacing at vf
        r = np.ldexp(np.rint(np.ldexp(vf, -q)), q)  # np.rint: halves go to the even integer
        out[fin] = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, r), r)
    return out


def fma_f32(a, b, c):
    """binary32 fused multiply-add: a*b + c rounded once to the nearest binary32 (ties to
    even), for binary32 inputs. The product of two binary32 values is exact in binary64;
    the binary64 sum is rounded to odd (its last bit set whenever the sum was inexact,
    found with the exact error term of the two-sum algorithm), and a round-to-odd value
    with two or more extra bits rounds to the same binary32 as the exact sum (Boldo and
    Melquiond, "When double rounding is odd")."""
    a = np.asarray(a, dtype=np.float32).astype(np.float64)
    b = np.asarray(b, dtype=np.float32).astype(np.float64)
    c = np.asarray(c, dtype=np.float32).astype(np.float64)
    p = a * b
    s = p + c
    bb = s - p
    err = (p - (s - bb)) + (c - bb)                 # p + c = s + err exactly
    even = (np.asarray(s).view(np.int64) & 1) == 0
    fix = (err != 0) & even & np.isfinite(s)
    s = np.where(fix, np.nextafter(s, np.where(err > 0, np.inf, -np.inf)), s)
    return s.astype(np.float32)


def combine_fp32(weights, y, shared=None):
    """The canonical reduction of one chunk in binary32: for each token and column,
    acc = 0; acc = fma(w[t, j], y[t, j], acc) for j = 0 .. k-1 (the token's experts in
    ascending id); acc = acc + shared[t] when there is a shared expert. weights [n, k]
    binary32, y [n, k, d] binary32 (expert outputs, unweighted), shared [n, d] or None.
    Returns acc [n, d] binary32 (before the final rounding to the storage type)."""
    w = np.asarray(weights, dtype=np.float32)
    y = np.asarray(y, dtype=np.float32)
    n, k = w.shape
    acc = np.zeros((n, y.shape[2]), dtype=np.float32)
    for j in range(k):
        acc = fma_f32(w[:, j, None], y[:, j, :], acc)
    if shared is not None:
        acc = acc + np.asarray(shared, dtype=np.float32)   # binary32 addition, one rounding
    return acc


# ---------------------------------------------------------------- bookkeeping

def member_lists(ids, n_experts):
    """Expert-major member lists of one chunk (token indices local to the chunk).

    counts[e]   rows routed to expert e
    offsets[e]  first row of expert e (exclusive prefix sum, offsets[E] = n*k)
    row_tok[r]  token of row r; rows of one expert are in ascending token order
    row_slot[r] t*k + j, where j is the position of e among token t's ascending ids
    """
    ids = np.asarray(ids)
    n, k = ids.shape
    counts = np.zeros(n_experts, dtype=np.int64)
    for e in ids.ravel():
        counts[e] += 1
    offsets = np.zeros(n_experts + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    row_tok = np.empty(n * k, dtype=np.int64)
    row_slot = np.empty(n * k, dtype=np.int64)
    fill = offsets[:-1].copy()
    for t in range(n):                      # tokens in ascending order
        for j in range(k):
            e = ids[t, j]
            row_tok[fill[e]] = t
            row_slot[fill[e]] = t * k + j
            fill[e] += 1
    return counts, offsets, row_tok, row_slot


def chunk_counts(ids, chunk, n_experts):
    """[ceil(T/chunk), E]: tokens of chunk c = [c*chunk, min((c+1)*chunk, T)) per expert."""
    ids = np.asarray(ids)
    T = ids.shape[0]
    n_chunks = (T + chunk - 1) // chunk
    out = np.zeros((n_chunks, n_experts), dtype=np.int64)
    for c in range(n_chunks):
        rows = ids[c * chunk: min((c + 1) * chunk, T)]
        out[c] = np.bincount(rows.ravel(), minlength=n_experts)
    return out


# ---------------------------------------------------------------- the layer

def moe_layer(x, params, ids=None):
    """One MoE layer over all rows of x [T, d] (the result is per token, so chunking does
    not change it).

    params: w_router [E, d], router_bias [E] or None, w_gu [E, 2I, d], w_down [E, d, I],
    w_gu_shared [2Is, d] or None, w_down_shared [d, Is] or None, top_k. Arrays may be bf16
    bit patterns (uint16) and are widened one expert at a time.
    ids: optional [T, k] expert ids to use instead of the oracle's own top-k (the routing
    gates substitute a set only where two logits are closer than the fp32 path can order).
    Returns dict(out [T, d], logits [T, E], ids [T, k], weights [T, k]).
    """
    x64 = as_f64(x)
    T, d = x64.shape
    k = int(params["top_k"])
    logits = router_logits(x64, params["w_router"], params.get("router_bias"))
    E = logits.shape[1]
    if ids is None:
        ids = select_topk(logits, k)
    ids = np.asarray(ids, dtype=np.int64)
    w = topk_weights(logits, ids)

    out = np.zeros((T, d), dtype=np.float64)
    for e in range(E):                      # ascending expert id
        t_idx, j_idx = np.nonzero(ids == e)
        if t_idx.size == 0:
            continue
        y = expert_ffn(x64[t_idx], params["w_gu"][e], params["w_down"][e])
        out[t_idx] += w[t_idx, j_idx][:, None] * y   # a token picks e at most once
    if params.get("w_gu_shared") is not None:
        out += expert_ffn(x64, params["w_gu_shared"], params["w_down_shared"])
    return {"out": out, "logits": logits, "ids": ids, "weights": w}


# ---------------------------------------------------------------- stack

def rmsnorm(x, eps):
    """x / sqrt(mean(x^2) + eps) per row (no gain)."""
    x = as_f64(x)
    return x / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + eps)


def moe_stack(x, layers, eps):
    """x <- x + layer_l(rmsnorm(x)) for each layer, float64 throughout."""
    x = as_f64(x)
    for p in layers:
        x = x + moe_layer(rmsnorm(x, eps), p)["out"]
    return x
