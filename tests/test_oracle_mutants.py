"""Planted mistakes in copies of the oracle: each must make at least one pin fail.

The mistakes are planted on the CPU, in fresh copies of the oracle module; the real oracle
is never modified.
"""
import importlib.util
import os

import numpy as np
import pytest

from tests.oracle_pins import ALL_PINS

_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                     "oracle", "moe_oracle.py")


def _fresh():
    spec = importlib.util.spec_from_file_location("_oracle_mutant", _PATH)
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def _m_ties_high(m):
    def select_topk(logits, k):
        logits = np.asarray(logits, dtype=np.float64)
        E = logits.shape[1]
        order = E - 1 - np.argsort(-logits[:, ::-1], axis=1, kind="stable")
        return np.sort(order[:, :k], axis=1)
    m.select_topk = select_topk


def _m_selection_order(m):
    def select_topk(logits, k):
        return np.argsort(-np.asarray(logits, dtype=np.float64), axis=1, kind="stable")[:, :k]
    m.select_topk = select_topk


def _m_no_renorm(m):
    def topk_weights(logits, ids):
        p = np.exp(logits - logits.max(axis=1, keepdims=True))
        p = p / p.sum(axis=1, keepdims=True)
        return np.take_along_axis(p, np.asarray(ids), axis=1)
    m.topk_weights = topk_weights


def _m_linear_weights(m):
    def topk_weights(logits, ids):
        c = np.take_along_axis(np.asarray(logits, dtype=np.float64), np.asarray(ids), axis=1)
        return c / c.sum(axis=1, keepdims=True)
    m.topk_weights = topk_weights


def _m_silu_sigmoid(m):
    m.silu = lambda z: 1.0 / (1.0 + np.exp(-z))


def _m_gate_up_swapped(m):
    def expert_ffn(xr, w_gu, w_down):
        xr = m.as_f64(xr); w_gu = m.as_f64(w_gu); inter = w_gu.shape[0] // 2
        up = xr @ w_gu[:inter].T; gate = xr @ w_gu[inter:].T
        return (m.silu(gate) * up) @ m.as_f64(w_down).T
    m.expert_ffn = expert_ffn


def _m_no_shared(m):
    orig = m.moe_layer
    def moe_layer(x, params, ids=None):
        p = dict(params); p["w_gu_shared"] = None
        return orig(x, p, ids)
    m.moe_layer = moe_layer


def _m_no_bias(m):
    orig = m.router_logits
    m.router_logits = lambda x, w, bias=None: orig(x, w, None)


def _m_reversed_slot_weights(m):
    orig = m.topk_weights
    m.topk_weights = lambda logits, ids: orig(logits, ids)[:, ::-1]


def _m_eps_outside(m):
    def rmsnorm(x, eps):
        x = m.as_f64(x)
        return x / (np.sqrt(np.mean(x * x, axis=1, keepdims=True)) + eps)
    m.rmsnorm = rmsnorm


def _m_no_residual(m):
    def moe_stack(x, layers, eps):
        x = m.as_f64(x)
        for p in layers:
            x = m.moe_layer(m.rmsnorm(x, eps), p)["out"]
        return x
    m.moe_stack = moe_stack


def _m_norm_after(m):
    def moe_stack(x, layers, eps):
        x = m.as_f64(x)
        for p in layers:
            x = x + m.rmsnorm(m.moe_layer(x, p)["out"], eps)
        return x
    m.moe_stack = moe_stack


def _m_member_desc(m):
    orig = m.member_lists
    def member_lists(ids, n_experts):
        counts, offsets, row_tok, row_slot = orig(ids, n_experts)
        for e in range(n_experts):
            a, b = offsets[e], offsets[e + 1]
            row_tok[a:b] = row_tok[a:b][::-1].copy(); row_slot[a:b] = row_slot[a:b][::-1].copy()
        return counts, offsets, row_tok, row_slot
    m.member_lists = member_lists


def _m_chunk_off_by_one(m):
    def chunk_counts(ids, chunk, n_experts):
        ids = np.asarray(ids); T = ids.shape[0]; n = (T + chunk - 1) // chunk
        out = np.zeros((n, n_experts), dtype=np.int64)
        for c in range(n):
            rows = ids[c * chunk + (1 if c else 0): min((c + 1) * chunk + 1, T)]
            out[c] = np.bincount(rows.ravel(), minlength=n_experts)
        return out
    m.chunk_counts = chunk_counts


def _m_widen_shift(m):
    orig = m.as_f64
    def as_f64(a):
        a2 = np.asarray(a) if a is not None else None
        if a2 is not None and a2.dtype == np.uint16:
            return (a2.astype(np.uint32) << 15).view(np.float32).astype(np.float64)
        return orig(a)
    m.as_f64 = as_f64


def _m_margin_index(m):
    def topk_margin(logits, k):
        srt = -np.sort(-np.asarray(logits, dtype=np.float64), axis=1)
        return srt[:, 0] - srt[:, min(k, srt.shape[1] - 1)]
    m.topk_margin = topk_margin


def _m_down_transposed_square(m):
    def expert_ffn(xr, w_gu, w_down):
        xr = m.as_f64(xr); w_gu = m.as_f64(w_gu); inter = w_gu.shape[0] // 2
        h = m.silu(xr @ w_gu[:inter].T) * (xr @ w_gu[inter:].T)
        wd = m.as_f64(w_down)
        return h @ wd.reshape(wd.shape[1], wd.shape[0])      # wrong orientation, right size
    m.expert_ffn = expert_ffn


def _m_bf16_ties_away(m):
    def bf16_rne(v):
        v = np.array(v, dtype=np.float64, copy=True)
        fin = np.isfinite(v) & (v != 0)
        _, e = np.frexp(v[fin]); q = np.maximum(e - 8, -133)
        s_ = np.ldexp(v[fin], -q)
        v[fin] = np.ldexp(np.sign(s_) * np.floor(np.abs(s_) + 0.5), q)
        return v
    m.bf16_rne = bf16_rne


def _m_bf16_truncate(m):
    def bf16_rne(v):
        v = np.array(v, dtype=np.float64, copy=True)
        fin = np.isfinite(v) & (v != 0)
        _, e = np.frexp(v[fin]); q = np.maximum(e - 8, -133)
        v[fin] = np.ldexp(np.trunc(np.ldexp(v[fin], -q)), q)
        return v
    m.bf16_rne = bf16_rne


def _m_bf16_nine_bits(m):
    def bf16_rne(v):
        v = np.array(v, dtype=np.float64, copy=True)
        fin = np.isfinite(v) & (v != 0)
        _, e = np.frexp(v[fin]); q = np.maximum(e - 9, -133)
        v[fin] = np.ldexp(np.rint(np.ldexp(v[fin], -q)), q)
        return v
    m.bf16_rne = bf16_rne


def _m_fma_unfused(m):
    def fma_f32(a, b, c):
        p = (np.asarray(a, dtype=np.float32) * np.asarray(b, dtype=np.float32)).astype(np.float32)
        return (p + np.asarray(c, dtype=np.float32)).astype(np.float32)
    m.fma_f32 = fma_f32


def _m_combine_descending(m):
    def combine_fp32(weights, y, shared=None):
        w = np.asarray(weights, dtype=np.float32); y = np.asarray(y, dtype=np.float32)
        acc = np.zeros((w.shape[0], y.shape[2]), dtype=np.float32)
        for j in reversed(range(w.shape[1])):
            acc = m.fma_f32(w[:, j, None], y[:, j, :], acc)
        if shared is not None:
            acc = acc + np.asarray(shared, dtype=np.float32)
        return acc
    m.combine_fp32 = combine_fp32


def _m_combine_shared_first(m):
    def combine_fp32(weights, y, shared=None):
        w = np.asarray(weights, dtype=np.float32); y = np.asarray(y, dtype=np.float32)
        acc = np.zeros((w.shape[0], y.shape[2]), dtype=np.float32)
        if shared is not None:
            acc = acc + np.asarray(shared, dtype=np.float32)
        for j in range(w.shape[1]):
            acc = m.fma_f32(w[:, j, None], y[:, j, :], acc)
        return acc
    m.combine_fp32 = combine_fp32


def _m_hidden_roles_swapped(m):
    def expert_hidden(xr, w_gu):
        xr = m.as_f64(xr); w_gu = m.as_f64(w_gu); inter = w_gu.shape[0] // 2
        up = xr @ w_gu[:inter].T; gate = xr @ w_gu[inter:].T
        return gate, up, m.silu(gate) * up
    m.expert_hidden = expert_hidden


MUTANTS = [v for k, v in sorted(globals().items()) if k.startswith("_m_")]


@pytest.mark.parametrize("mutate", MUTANTS, ids=[f.__name__[3:] for f in MUTANTS])
def test_planted_mistake_is_caught(mutate):
    m = _fresh()
    mutate(m)
    failed = []
    for pin in ALL_PINS:
        try:
            pin(m)
        except Exception:           # an assertion or a shape error both count as caught
            failed.append(pin.__name__)
    assert failed, f"no pin catches {mutate.__name__}"
