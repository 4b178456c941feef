"""Seeded random layer shapes: for each, every chunking gives the batched pass's bytes, the
fused routed launch (where its 64-row tiles apply) gives the same bytes again, and the batched
chunk passes the element-wise stage checks against the oracle (h and h_shared at their
rounding, Y within its fp32 bound, out at its rounding). The shapes cover expert counts that
are not multiples of 64, k = 1, no shared expert, one-token prompts, uneven last chunks and
every routed tile height."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
from tests import test_gpu_stages as st
from tests.parity import oracle_params, place

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


def _shape(seed):
    rng = np.random.default_rng(seed)
    E = int(rng.choice([2, 3, 8, 17, 33, 64, 130, 257]))
    k = int(rng.integers(1, min(8, E) + 1))
    T = int(rng.choice([1, 7] + [int(t) for t in rng.integers(16, 3000, size=4)]))
    kw = dict(T=T, d=int(64 * rng.integers(1, 9)), E=E, k=k, inter=int(128 * rng.integers(1, 5)),
              inter_shared=int(64 * rng.integers(0, 9)),
              zipf_s=[None, 1.1, 1.5][int(rng.integers(0, 3))], seed=2000 + seed)
    chunks = sorted(set(int(c) for c in rng.integers(1, T + 1, size=3)))
    return kw, chunks


@pytest.mark.parametrize("seed", range(20))
def test_random_shape(moe, seed):
    kw, chunks = _shape(seed)
    print(f"[random] seed {seed}: {kw} chunks {chunks}", flush=True)
    wl = mi.custom_workload("random", **kw)
    params, L = place(wl)
    x = mi.make_x(wl, device="cuda")
    base = moe.moe_prefill_layer(L, x, wl.T)
    torch.cuda.synchronize()
    ref = base["out"].clone()
    for fused in (0, 1):
        moe.moe_set_option("fused_gu_down", fused)
        try:
            for c in chunks:
                got = moe.moe_prefill_layer(L, x, c)
                torch.cuda.synchronize()
                assert torch.equal(bits(got["out"]), bits(ref)), (c, fused)
        finally:
            moe.moe_set_option("fused_gu_down", 0)
    c = st.Chunk(moe, wl, params, x, 0, wl.T)
    op = oracle_params(params, wl)
    stats = st._new_stats()
    st._check_routed(c, op, range(wl.shape.n_experts), stats)
    st._check_out(c, op, np.arange(wl.T), stats)
    print(f"[random] seed {seed}: h {stats['h'][1]}/{stats['h'][0]} out {stats['out'][1]}/"
          f"{stats['out'][0]} decided, Y worst err/bound {stats['y_worst']:.3g}", flush=True)
    for key in ("h", "out"):
        n_, dec, _ = stats[key]
        assert dec >= st.MIN_DECIDED * n_, (key, dec, n_)
