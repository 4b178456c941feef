"""HIP path against the fp64 oracle (element by element) and against itself across chunk
sizes, through the C ABI. Needs an MI355X."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle.moe_oracle as orc
from tests.parity import as_f64, logit_bound, oracle_params, place, rel_err, routing_gates

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2     # max-abs error over output RMS, bf16 outputs
F32_TOL = 1e-4      # same metric, fp32 storage and arithmetic


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import routed_expert_grouped_moe_amd as m
    m.moe_abi_version()
    return m


def bits(t):
    """Bit patterns of a tensor (compares NaNs and signed zeros exactly)."""
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _run(moe, L, x, chunk, **kw):
    r = moe.moe_prefill_layer(L, x, chunk, **kw)
    torch.cuda.synchronize()
    return r


def _full_parity(moe, wl, tol, chunks=None):
    """Whole-layer parity against the oracle plus bit-identity across chunk sizes."""
    params, L = place(wl)
    x = mi.make_x(wl, device="cuda")
    chunks = chunks or wl.chunks
    outs = {}
    for c in chunks:
        outs[c] = _run(moe, L, x, c)
    base = outs[chunks[-1]]
    for c in chunks:
        assert torch.equal(bits(outs[c]["out"]), bits(base["out"])), f"chunk {c}"
        assert torch.equal(outs[c]["ids"], base["ids"])
    op = oracle_params(params, wl)
    xh = mi.to_numpy_exact(x)
    ref_logits = orc.router_logits(xh, op["w_router"], op["router_bias"])
    bound = logit_bound(xh, op["w_router"], ref_logits, wl.shape.dtype)
    ids_use, ties = routing_gates(base["logits"].cpu().numpy(), base["ids"].cpu().numpy(),
                                  base["weights"].cpu().numpy(), ref_logits, wl.shape.top_k,
                                  bound)
    for c in chunks:
        cc = outs[c]["chunk_counts"].cpu().numpy()
        assert np.array_equal(cc, orc.chunk_counts(outs[c]["ids"].cpu().numpy(), c,
                                                   wl.shape.n_experts)), f"counts, chunk {c}"
    ref = orc.moe_layer(xh, op, ids=ids_use)["out"]
    err = rel_err(as_f64(base["out"]), ref)
    print(f"{wl.name}: rel err {err:.3e}, near-ties {ties}")
    if tol is not None:
        assert err <= tol, err
    return err


def test_tiny_fp32(moe):
    _full_parity(moe, mi.WORKLOADS["tiny_fp32"], F32_TOL, chunks=(40, 7, 1))


def test_fp32_tile_heights_and_deferred_combine(moe):
    """fp32 storage through the 256-, 128- and 64-row routed tiles (E = 16, k = 4: 600 tokens
    batched and 520-token chunks take 256-row tiles, 200-token chunks 128-row ones, 64-token
    chunks and the 80-token tail 64-row ones, a 24-token tail 16-row ones), each chunked call
    deferring its shared down + combine into the next chunk's gate/up launch: the batched
    bytes at every chunk size, and oracle parity."""
    wl = mi.custom_workload("f32_tiles", T=600, d=128, E=16, k=4, inter=64, inter_shared=128,
                            dtype="f32", zipf_s=1.1, seed=5)
    _full_parity(moe, wl, F32_TOL, chunks=(64, 200, 520, 600))


@pytest.mark.parametrize("dtype,tol", [("f32", F32_TOL), ("bf16", None)])
def test_short_prompt_shared_tiles(moe, dtype, tol):
    """Chunks averaging fewer than 16 rows per expert (E = 64, k = 2: up to 511 tokens) of
    more than 192 tokens run the shared expert's GEMMs in launches of their own, here on 64x64
    tiles (300 tokens); smaller ones run them inside the routed launches as 16-row blocks (100
    and 40 tokens). All give the same bytes, and in fp32 the oracle's values. (bf16 at
    d = 128: the end-to-end error gate is left to the wider layers and the stage checks;
    routing is still gated.)"""
    wl = mi.custom_workload("short_" + dtype, T=300, d=128, E=64, k=2, inter=64,
                            inter_shared=128, dtype=dtype, zipf_s=1.1, seed=29)
    _full_parity(moe, wl, tol, chunks=(40, 100, 300))


def test_small_bf16_many_chunks(moe):
    wl = mi.custom_workload("small", T=300, d=128, E=16, k=4, inter=64, inter_shared=128,
                            zipf_s=1.1, seed=3)
    _full_parity(moe, wl, BF16_TOL, chunks=(1, 3, 7, 64, 129, 300))


@pytest.mark.parametrize("case", [
    dict(T=37, d=64, E=1, k=1, inter=64, inter_shared=64),        # a single expert
    dict(T=50, d=128, E=8, k=8, inter=64, inter_shared=0),         # k = E, no shared expert
    dict(T=1, d=256, E=32, k=3, inter=128, inter_shared=64),       # one token
    dict(T=515, d=192, E=200, k=6, inter=192, inter_shared=192),   # E not a multiple of 64/128
    dict(T=260, d=64, E=1024, k=2, inter=64, inter_shared=0),      # largest E
])
def test_edge_shapes(moe, case):
    wl = mi.custom_workload("edge", seed=11, **case)
    chunks = (max(1, case["T"] // 3), case["T"])
    _full_parity(moe, wl, BF16_TOL, chunks=chunks)


@pytest.mark.parametrize("case", [
    dict(T=33, d=16384, E=4, k=2, inter=64, inter_shared=64),      # largest d
    dict(T=33, d=64, E=4, k=2, inter=16384, inter_shared=0),       # largest I
    dict(T=33, d=64, E=2, k=1, inter=64, inter_shared=65536),      # largest I_s
])
def test_largest_dims(moe, case):
    """Each of d, I and I_s at the largest value the header allows (the others small, so the
    oracle stays cheap): 256 to 1,024 K stages per tile and up to 128 N-units per expert.
    Gaussian layer: routing against the oracle, chunks of 11 (decode tiles) and 33 tokens
    bit-identical (the whole-tensor error is printed, not gated: with two terms per output it
    measures the bf16 roundings themselves). Small-integer layer of the same shape: every
    stage bit for bit, at both chunkings. (At K = 16,384 the Gaussian stage bound spans most
    bf16 roundings of h, so only the exact layer can tell a right GEMM from a wrong one.)"""
    from tests import test_gpu_stages as st
    wl = mi.custom_workload("maxdim", seed=12, **case)
    print(f"[maxdim] {case}", flush=True)
    _full_parity(moe, wl, None, chunks=(11, 33))
    params = mi.make_int_layer(wl, device="cuda")
    x = mi.make_int_x(wl, device="cuda")
    for t0, n in ((0, 11), (0, 33)):
        st._int_bit_exact(moe, wl, params, x, t0, n, sample=None)


def test_k_above_64(moe):
    """k = 100 of E = 130 experts: top-k rounds past the first 64, the bucketing's check of a
    token's later slots against its earlier ids (slots 64 and up), and combines of 100 terms.
    Routing, chunks of 1, 13 and 40 tokens bit-identical, element-wise stage parity."""
    wl = mi.custom_workload("k100", T=40, d=128, E=130, k=100, inter=64, inter_shared=64,
                            seed=13)
    _full_parity(moe, wl, BF16_TOL, chunks=(1, 13, 40))
    _stage_parity(moe, wl)


def _stage_parity(moe, wl):
    """Element-wise stage parity of the batched pass (tests/stage_checks.py): h, Y and out
    of every expert and token against the oracle's stages within derived bounds. Used where
    the whole-tensor max-abs/RMS metric is dominated by the bf16 roundings themselves (few
    terms per output, skewed routing): an ideal bf16 pipeline scores 1.5e-2 to 2.8e-2 on
    such shapes, so that metric cannot tell a right kernel from a slightly wrong one."""
    from tests import test_gpu_stages as st
    params = mi.make_layer(wl, device="cuda")
    x = mi.make_x(wl, device="cuda")
    c = st.Chunk(moe, wl, params, x, 0, wl.T)
    op = oracle_params(params, wl)
    stats = st._new_stats()
    st._check_routed(c, op, range(wl.shape.n_experts), stats)
    st._check_out(c, op, np.arange(wl.T), stats)
    st._report(wl.name, stats)


def test_big_tiles_with_partial_tiles(moe):
    """A chunk averaging at least 128 rows per expert takes 256-row M-tiles; an expert's
    remainder gets one more, partly filled tile. The seeded routing hits the cases (experts
    with fewer than 64 rows, small remainders after full tiles, several full tiles plus a
    large partial one). Element-wise stage parity with the oracle, and the bytes equal those
    of the all-64-row tiling that a 100-token chunk takes."""
    wl = mi.custom_workload("tails", T=2000, d=128, E=16, k=4, inter=128, inter_shared=256,
                            zipf_s=1.1, seed=15)
    params, L = place(wl)
    x = mi.make_x(wl, device="cuda")
    r = moe.moe_prefill_route(L, x, wl.T)
    torch.cuda.synchronize()
    c = r["chunk_counts"][0].cpu().numpy()
    assert wl.T * wl.shape.top_k >= wl.shape.n_experts * 128      # 256-row tiling
    rem = c % 256
    assert ((c > 0) & (c <= 64)).any()
    assert ((c > 256) & (rem > 0) & (rem <= 64)).any() and ((c > 512) & (rem > 64)).any()
    _chunks_identical(moe, wl, (100, wl.T))
    _stage_parity(moe, wl)


def _chunks_identical(moe, wl, chunks):
    params, L = place(wl)
    x = mi.make_x(wl, device="cuda")
    outs = [_run(moe, L, x, c)["out"].clone() for c in chunks]
    for c, o in zip(chunks[1:], outs[1:]):
        assert torch.equal(bits(o), bits(outs[0])), f"chunk {c} against chunk {chunks[0]}"


def test_tall_tiles(moe):
    """A chunk averaging 192 to 320 rows per expert takes 320-row M-tiles (8 waves of 80 x 128):
    an expert of 257..320 rows fits one tile. The seeded routing has experts above 320 rows
    (several tiles), of 257..320 rows, of about 200 rows (the last wave slab idle) and under
    80 rows (the seed is one whose routing covers all four cases). Element-wise stage parity
    with the oracle, and the bytes equal those of the 64-row tiling of a 100-token chunk."""
    wl = mi.custom_workload("tall", T=1000, d=256, E=16, k=4, inter=128, inter_shared=256,
                            zipf_s=1.1, seed=32)
    params, L = place(wl)
    x = mi.make_x(wl, device="cuda")
    r = moe.moe_prefill_route(L, x, wl.T)
    torch.cuda.synchronize()
    c = r["chunk_counts"][0].cpu().numpy()
    rows, E = wl.T * wl.shape.top_k, wl.shape.n_experts
    assert 192 * E <= rows < 320 * E                               # 320-row tiling
    assert (c > 320).any() and ((c > 256) & (c <= 320)).any() and ((c > 0) & (c < 80)).any()
    _chunks_identical(moe, wl, (100, wl.T))
    _stage_parity(moe, wl)


def test_topk_ties_and_special_values(moe):
    """Top-k on logits with exact ties (duplicated router rows), NaN and -inf (from the bias),
    an all-NaN token and a zero token, with E = 130 (ragged lane slices). The ids equal the
    oracle's selection on the GPU's own logits with NaN read as -inf (lower id first among
    equal values); the weights match the oracle's to fp32 rounding."""
    wl = mi.custom_workload("topk", T=200, d=64, E=130, k=5, inter=64, inter_shared=0,
                            zipf_s=1.1, seed=21)
    p = mi.make_layer(wl, 0, device="cuda")
    w, b = p["w_router"], p["router_bias"]
    w[10:20] = w[10].clone()
    w[100:130] = w[3].clone()
    b.zero_()
    b[50] = float("nan")
    b[51] = float("-inf")
    b[60] = 30.0
    params, L = place(wl, params=p)
    x = mi.make_x(wl, device="cuda")
    x[7] = float("nan")
    x[8] = 0
    r = moe.moe_prefill_route(L, x, 64)
    torch.cuda.synchronize()
    logits = r["logits"].cpu().numpy().astype(np.float64)
    lg = np.where(np.isnan(logits), -np.inf, logits)
    ids = r["ids"].cpu().numpy()
    assert np.array_equal(ids, orc.select_topk(lg, wl.shape.top_k))
    assert list(ids[7]) == [0, 1, 2, 3, 4]          # every logit NaN: five lowest ids
    assert list(ids[8]) == [0, 1, 2, 3, 60]         # logits = bias: 30, then ties at 0
    assert np.all(np.isin(ids, [50, 51], invert=True)[np.arange(wl.T) != 7])
    ok = ~np.isnan(logits).all(axis=1)
    wts = r["weights"].cpu().numpy()
    w_ref = orc.topk_weights(lg[ok], ids[ok])
    assert np.max(np.abs(w_ref - wts[ok])) <= 2e-6
    assert np.array_equal(r["chunk_counts"].cpu().numpy(),
                          orc.chunk_counts(ids, 64, wl.shape.n_experts))
    # chunk 1: a 256-token block spans more (chunk, expert) bins than its LDS histogram holds
    r1 = moe.moe_prefill_route(L, x, 1)
    torch.cuda.synchronize()
    assert np.array_equal(r1["ids"].cpu().numpy(), ids)
    assert np.array_equal(r1["chunk_counts"].cpu().numpy(),
                          orc.chunk_counts(ids, 1, wl.shape.n_experts))


def test_member_lists_bit_exact(moe):
    """The GPU's expert-major member lists equal the oracle's, integer for integer, for chunks
    of one to twenty 256-token blocks (up to 8 blocks the scan runs inside the permute kernel,
    above that in a kernel of its own)."""
    wl = mi.custom_workload("lists", T=5000, d=128, E=16, k=4, inter=64, inter_shared=64,
                            zipf_s=1.5, seed=5)
    params, L = place(wl)
    x = mi.make_x(wl, device="cuda")
    sh = L.shape
    r = moe.moe_prefill_route(L, x, 300)
    out = torch.empty_like(x)
    for t0, n in ((0, 300), (300, 300), (900, 100), (900, 2048), (400, 2600), (0, 4096),
                  (0, 5000)):
        ws = torch.empty(moe.moe_workspace_bytes(sh, n), dtype=torch.uint8, device="cuda")
        moe.moe_prefill_chunk(L, x, r["ids"], r["weights"], t0, n, out, ws)
        torch.cuda.synchronize()
        off = moe.moe_workspace_offsets(sh, n)
        w8 = ws.cpu().numpy()
        as_i32 = lambda o, cnt: w8[o: o + 4 * cnt].view(np.int32)
        counts, offsets, row_tok, row_slot = orc.member_lists(
            r["ids"][t0:t0 + n].cpu().numpy(), sh.n_experts)
        assert np.array_equal(as_i32(off["counts"], sh.n_experts), counts)
        assert np.array_equal(as_i32(off["offsets"], sh.n_experts + 1), offsets)
        assert np.array_equal(as_i32(off["row_tok"], n * sh.top_k), row_tok)
        assert np.array_equal(as_i32(off["row_slot"], n * sh.top_k), row_slot)


def test_invalid_ids_are_dropped(moe):
    """Caller-provided ids with a slot out of range or repeated within a token: the bucketing
    drops those slots alike in every kernel, the resident call completes, and every other
    token keeps the bytes it gets with valid ids, both when the scan runs inside the permute
    kernel (3 token blocks) and in its own kernel (10 blocks). With a ring the counts fall short
    of n*k and the call fails with MOE_ERR_INVALID, leaving out unchanged."""
    wl = mi.custom_workload("badids", T=2500, d=128, E=16, k=4, inter=64, inter_shared=64,
                            seed=27)
    params, L = place(wl)
    x = mi.make_x(wl, device="cuda")
    sh = L.shape
    r = moe.moe_prefill_route(L, x, wl.T)
    bad = r["ids"].clone()
    bad[5, 1] = sh.n_experts            # one past the last expert
    bad[6, 2] = -3
    bad[7, 3] = bad[7, 0]               # repeated expert
    bad[300, 0] = 1 << 20
    bad[2400, :] = bad[2400, 0]         # every slot the same expert
    hit = [5, 6, 7, 300, 2400]
    for n in (600, wl.T):
        ws = torch.empty(moe.moe_workspace_bytes(sh, n), dtype=torch.uint8, device="cuda")
        ref = torch.zeros_like(x)
        moe.moe_prefill_chunk(L, x, r["ids"], r["weights"], 0, n, ref, ws)
        got = torch.zeros_like(x)
        moe.moe_prefill_chunk(L, x, bad, r["weights"], 0, n, got, ws)
        torch.cuda.synchronize()
        keep = torch.ones(wl.T, dtype=torch.bool, device="cuda")
        keep[n:] = False
        keep[hit] = False
        assert torch.equal(bits(got[keep]), bits(ref[keep])), n
    ring = moe.Ring(sh, 8)
    _, Lr = place(wl, offloaded=range(sh.n_experts), ring=ring, params=params)
    ws = torch.empty(moe.moe_workspace_bytes(sh, 600), dtype=torch.uint8, device="cuda")
    out = torch.zeros_like(x)
    with pytest.raises(moe.MoeError, match="MOE_ERR_INVALID"):
        moe.moe_prefill_chunk(Lr, x, bad, r["weights"], 0, 600, out, ws)
    torch.cuda.synchronize()
    assert not out.any()
    ring.close()


def test_repeatable_five_runs(moe):
    wl = mi.custom_workload("rep", T=700, d=256, E=64, k=6, inter=128, inter_shared=256,
                            zipf_s=1.1, seed=9)
    params, L = place(wl)
    x = mi.make_x(wl, device="cuda")
    first = _run(moe, L, x, 256)
    for _ in range(4):
        again = _run(moe, L, x, 256)
        assert torch.equal(bits(again["out"]), bits(first["out"]))
        assert torch.equal(again["logits"], first["logits"])
        assert torch.equal(again["weights"], first["weights"])


def test_row_position_invariance(moe):
    """A token's bytes do not depend on its position: permuting the prompt permutes the output."""
    wl = mi.custom_workload("perm", T=333, d=128, E=16, k=4, inter=128, inter_shared=64, seed=4)
    params, L = place(wl)
    x = mi.make_x(wl, device="cuda")
    perm = torch.randperm(wl.T, generator=torch.Generator().manual_seed(0)).cuda()
    a = _run(moe, L, x, 100)["out"]
    b = _run(moe, L, x[perm].contiguous(), 64)["out"]
    assert torch.equal(bits(b), bits(a[perm]))


def test_workspace_too_small_leaves_output(moe):
    wl = mi.custom_workload("ws", T=64, d=128, E=8, k=2, inter=64, inter_shared=64)
    params, L = place(wl)
    x = mi.make_x(wl, device="cuda")
    r = moe.moe_prefill_route(L, x, 64)
    out = torch.full_like(x, 3.0)
    ws = torch.empty(moe.moe_workspace_bytes(L.shape, 64) - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(moe.MoeError, match="MOE_ERR_WORKSPACE"):
        moe.moe_prefill_chunk(L, x, r["ids"], r["weights"], 0, 64, out, ws)
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)
    # a smaller chunk fits the same workspace and gives the same bytes as the batched pass
    full = _run(moe, L, x, 64)["out"]
    for t0 in range(0, 64, 32):
        moe.moe_prefill_chunk(L, x, r["ids"], r["weights"], t0, 32, out, ws)
    torch.cuda.synchronize()
    assert torch.equal(bits(out), bits(full))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_router_logits_independent_of_tile_shape(moe, dtype):
    """The router GEMM picks its tile (256 or 128 rows; 64 rows by 256 columns with two or four
    stage buffers; 64 by 64; 16 by 16) from T; a token's logits, and so its routing, are the
    same bytes whichever tile computed them."""
    wl = mi.custom_workload("rtile", T=49152, d=256, E=512, k=8, inter=64, inter_shared=0,
                            dtype=dtype, seed=23)
    params, L = place(wl)
    x = mi.make_x(wl, device="cuda")
    ref = moe.moe_prefill_route(L, x, 49152)      # 192 x 2 = 384 tiles of 256 rows
    # 128 rows; 64 x 256 (2 and 4 buffers); 64 x 64; 16 x 16 (3 row blocks, and one)
    for T in (12288, 10000, 6000, 700, 40, 9):
        got = moe.moe_prefill_route(L, x[:T].contiguous(), T)
        torch.cuda.synchronize()
        for key in ("logits", "ids", "weights"):
            assert torch.equal(bits(ref[key][:T]), bits(got[key])), (T, key)


def test_layer_3001(moe):
    """bf16 layer, T = 3,001, all experts resident: deep chunk 1,024 equals the batched pass
    bit for bit, and both match the oracle."""
    _full_parity(moe, mi.WORKLOADS["layer_3001"], BF16_TOL)


def test_row_path_equals_batched(moe):
    """The single-row path (a chunk of one token, as a decoder would run it, on the same
    kernels) gives each token the bytes of the batched pass, at the full layer size."""
    wl = mi.WORKLOADS["layer_3001"]
    params, L = place(wl)
    x = mi.make_x(wl, device="cuda")
    base = _run(moe, L, x, wl.T)
    sh = L.shape
    ws = torch.empty(moe.moe_workspace_bytes(sh, 1), dtype=torch.uint8, device="cuda")
    out = torch.zeros_like(x)
    rows = [0, 1, 1500, 2999, wl.T - 1]
    for t in rows:
        moe.moe_prefill_chunk(L, x, base["ids"], base["weights"], t, 1, out, ws)
    torch.cuda.synchronize()
    for t in rows:
        assert torch.equal(bits(out[t]), bits(base["out"][t])), t


def test_decode_sized_call_equals_batched(moe):
    """A call of a few tokens runs every GEMM on the 16-row decode tiles; each token gets the
    bytes the batched pass gives it, routing included."""
    wl = mi.WORKLOADS["layer_3001"]
    params, L = place(wl)
    x = mi.make_x(wl, device="cuda")
    base = _run(moe, L, x, wl.T)
    E = wl.shape.n_experts
    for t0, n, chunk in ((0, 1, 1), (5, 8, 8), (2990, 11, 11), (100, 16, 5)):
        xs = x[t0:t0 + n].contiguous()
        got = _run(moe, L, xs, chunk)
        torch.cuda.synchronize()
        ids = got["ids"].cpu().numpy()
        assert torch.equal(got["ids"], base["ids"][t0:t0 + n]), (t0, n)
        assert torch.equal(bits(got["out"]), bits(base["out"][t0:t0 + n])), (t0, n)
        # per-chunk counts (the top-k of at most 16 tokens counts them in the same launch)
        want = np.stack([np.bincount(ids[c:c + chunk].ravel(), minlength=E)
                         for c in range(0, n, chunk)])
        assert np.array_equal(got["chunk_counts"].cpu().numpy(), want), (t0, n, chunk)


def test_chunk_gate_4099(moe):
    """Zipf(1.1)-skewed routing, T = 4,099: chunks 256 / 1,024 / 2,048 and the batched pass
    give identical bytes."""
    _full_parity(moe, mi.WORKLOADS["chunk_gate_4099"], BF16_TOL)


def test_add_rmsnorm(moe):
    g = torch.Generator(device="cuda").manual_seed(3)
    x = torch.randn(77, 2048, device="cuda", generator=g).to(torch.bfloat16)
    dlt = torch.randn(77, 2048, device="cuda", generator=g).to(torch.bfloat16)
    xn, nrm = moe.moe_add_rmsnorm(x, dlt, 1e-6)
    torch.cuda.synchronize()
    # residual add: one rounding of the exact sum (torch's own bf16 rounding is the reference)
    want = (x.double() + dlt.double()).to(torch.bfloat16)
    assert torch.equal(xn.view(torch.int16), want.view(torch.int16))
    # normed: fp32 arithmetic then one bf16 rounding, so each element is within half a bf16
    # ulp (2^-9 relative) of the exact value, plus fp32 noise; 2^-8 relative bounds both
    ref = orc.rmsnorm(as_f64(xn), 1e-6)
    assert np.all(np.abs(as_f64(nrm) - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-30)
    # without delta: normalise only; in place form
    _, n2 = moe.moe_add_rmsnorm(x, None, 1e-6)
    ref2 = orc.rmsnorm(as_f64(x), 1e-6)
    assert np.all(np.abs(as_f64(n2) - ref2) <= 2.0 ** -8 * np.abs(ref2) + 1e-30)
    x2 = x.clone()
    moe.moe_add_rmsnorm(x2, dlt, 1e-6, x_out=x2)
    torch.cuda.synchronize()
    assert torch.equal(x2.view(torch.int16), want.view(torch.int16))


@pytest.mark.parametrize("T,chunk,alone", [(3001, 1024, 1), (700, 256, 1), (900, 200, 1),
                                           (16022, 4096, 1), (6096, 4096, 2), (1800, 800, 1)])
def test_prebucketed_layer_equals_per_chunk(moe, T, chunk, alone):
    """A layer call whose workspace holds every chunk's member lists buckets all chunks in one
    set of launches and defers each chunk's shared down + combine to the next chunk's gate/up
    launch where both chunks' tiles allow; with the base workspace each chunk buckets before
    its own GEMMs and runs its own shared down + combine. Same output bytes and chunk counts
    either way (and the batched pass's bytes). E = 64, k = 8: 1,024- and 4,096-token chunks
    take 256-row tiles (down units last), a last chunk of 953 tokens 128-row ones, 256 and 200
    tokens 64-row ones (down units first; 800-token chunks take 128-row tiles and hand their
    shared down + combine to a 200-token last chunk on 64-row tiles); a last chunk of 100
    tokens (16-row tiles, its shared expert inside the routed launches and the stand-alone
    combine after them) and one of 2,000 (320-row tiles) cannot take the deferred launch, which
    then runs alone before them (`alone`: stand-alone shared down + combine launches of the
    layer call). Also one-block
    chunks, chunks of 200 tokens that straddle token blocks, and the separate scan launch
    (4,096-token chunks: 16 blocks)."""
    wl = mi.custom_workload("prebucket", T=T, d=256, E=64, k=8, inter=128, inter_shared=256,
                            zipf_s=1.1, seed=41)
    print(f"[prebucket] T={T} chunk={chunk}", flush=True)
    _, L = place(wl)
    x = mi.make_x(wl, device="cuda")
    bufs = moe.layer_buffers(L, T, chunk)
    assert bufs["workspace"].numel() > moe.moe_workspace_bytes(L.shape, chunk)
    moe.moe_profile_read(reset=True)
    moe.moe_profile_enable(True)
    try:
        a = moe.moe_prefill_layer(L, x, chunk, bufs=bufs)
        torch.cuda.synchronize()
    finally:
        moe.moe_profile_enable(False)
    prof = moe.moe_profile_read(reset=True)
    out_a, cc_a = a["out"].clone(), a["chunk_counts"].clone()
    n_chunks = (T + chunk - 1) // chunk
    assert prof["permute"][1] == 1                                 # one launch, every chunk
    assert prof["down_shared_combine"][1] == alone
    assert prof["gu_mixed"][1] + prof["gu_shared"][1] == n_chunks
    small = dict(bufs)
    small["workspace"] = torch.empty(moe.moe_workspace_bytes(L.shape, chunk), dtype=torch.uint8,
                                     device="cuda")
    moe.moe_profile_enable(True)
    try:
        b = moe.moe_prefill_layer(L, x, chunk, bufs=small)
        torch.cuda.synchronize()
    finally:
        moe.moe_profile_enable(False)
    prof = moe.moe_profile_read(reset=True)
    assert prof["permute"][1] == n_chunks                         # one per chunk
    sizes = [min(chunk, T - t0) for t0 in range(0, T, chunk)]    # decode-sized: combine alone
    n_small = sum(n <= 192 and n * 8 < 16 * 64 for n in sizes)
    assert prof["down_shared_combine"][1] == n_chunks - n_small
    assert prof["combine"][1] == n_small
    assert torch.equal(bits(b["out"]), bits(out_a))
    assert torch.equal(b["chunk_counts"], cc_a)
    ref = _run(moe, L, x, T)["out"]
    assert torch.equal(bits(ref), bits(out_a))
    want = orc.chunk_counts(a["ids"].cpu().numpy(), chunk, wl.shape.n_experts)
    assert np.array_equal(cc_a.cpu().numpy(), want)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_tile_chunks_defer_shared_combine(moe, dtype):
    """Chunks on decode tiles (E = 64, k = 2: fewer than 512 tokens) of 193 to 512 tokens, in a
    layer call that buckets up front, run their shared gate/up as 16-row blocks inside their
    gate/up launch and leave their shared down + combine to the next chunk's: the 300-token
    chunks of a 1,100-token prompt and its 200-token tail launch one stand-alone shared down +
    combine (the last chunk's) and no stand-alone shared gate/up, the per-chunk path four of
    each, with the same bytes (and the batched pass's)."""
    wl = mi.custom_workload("ddefer", T=1100, d=256, E=64, k=2, inter=128, inter_shared=256,
                            dtype=dtype, zipf_s=1.1, seed=43)
    _, L = place(wl)
    x = mi.make_x(wl, device="cuda")
    T, chunk = wl.T, 300
    bufs = moe.layer_buffers(L, T, chunk)
    runs = {}
    for name, ws in (("layer", bufs["workspace"]),
                     ("per_chunk", torch.empty(moe.moe_workspace_bytes(L.shape, chunk),
                                               dtype=torch.uint8, device="cuda"))):
        b = dict(bufs)
        b["workspace"] = ws
        moe.moe_profile_read(reset=True)
        moe.moe_profile_enable(True)
        try:
            r = moe.moe_prefill_layer(L, x, chunk, bufs=b)
            torch.cuda.synchronize()
        finally:
            moe.moe_profile_enable(False)
        runs[name] = (r["out"].clone(), moe.moe_profile_read(reset=True))
    out_l, prof_l = runs["layer"]
    out_c, prof_c = runs["per_chunk"]
    assert prof_l["down_shared_combine"][1] == 1 and prof_l["gu_shared"][1] == 0
    assert prof_l["gu_mixed"][1] == 4
    assert prof_c["down_shared_combine"][1] == 4 and prof_c["gu_shared"][1] == 4
    assert torch.equal(bits(out_l), bits(out_c))
    assert torch.equal(bits(out_l), bits(_run(moe, L, x, T)["out"]))


def test_profile_times_and_clocks(moe):
    """The opt-in profiling counts every GEMM launch and samples a plausible shader clock for
    each GEMM stage; turning it off records nothing more. (Experts resident, so the shared
    and routed gate/up GEMMs share one launch per chunk.)"""
    wl = mi.custom_workload("prof", T=700, d=256, E=64, k=6, inter=128, inter_shared=256,
                            seed=9)
    params, L = place(wl)
    x = mi.make_x(wl, device="cuda")
    moe.moe_profile_read(reset=True)
    moe.moe_profile_enable(True)
    try:
        _run(moe, L, x, 256)
    finally:
        moe.moe_profile_enable(False)
    prof = moe.moe_profile_read(reset=True, clocks=True)
    for stage in ("router", "gu_mixed", "down_routed", "down_shared_combine"):
        ms, n, mhz = prof[stage]
        assert n >= 1 and ms > 0, (stage, prof[stage])
        assert 100 < mhz < 3500, (stage, mhz)
    # one gate/up launch per chunk; the first two chunks' shared down + combine run inside the
    # next chunk's, the last chunk's alone
    assert prof["down_shared_combine"][1] == 1 and prof["gu_mixed"][1] == 3
    assert prof["combine"][1] == 0 and prof["down_shared"][1] == 0  # folded together
    assert prof["gu_routed"][1] == 0 and prof["gu_shared"][1] == 0
    _run(moe, L, x, 256)
    assert all(v[1] == 0 for v in moe.moe_profile_read(reset=True).values())


def test_small_chunks_mix_the_shared_expert_in(moe):
    """Chunks on decode tiles (fewer than 16 rows per expert) of at most 192 tokens run the
    shared expert's tiles, as 16-row blocks, inside the routed gate/up and down launches and
    the stand-alone combine after them; larger chunks fold the combine into the shared down
    GEMM. Both give the batched pass's bytes. (E = 64, k = 2: decode tiles below 512 tokens;
    chunks of 5, 16, 17 and 192 tokens and a 108-token tail are mixed, 250 and 300 not; in a
    layer call the 250-token chunk defers its shared down + combine.)"""
    wl = mi.custom_workload("side", T=300, d=256, E=64, k=2, inter=128, inter_shared=256,
                            zipf_s=1.1, seed=19)
    params, L = place(wl)
    x = mi.make_x(wl, device="cuda")
    base = _run(moe, L, x, wl.T)
    for chunk in (16, 17, 5, 192, 250):
        moe.moe_profile_read(reset=True)
        moe.moe_profile_enable(True)
        try:
            got = _run(moe, L, x, chunk)
            torch.cuda.synchronize()
        finally:
            moe.moe_profile_enable(False)
        prof = moe.moe_profile_read(reset=True)
        sizes = [min(chunk, wl.T - t0) for t0 in range(0, wl.T, chunk)]
        decode = [n * wl.shape.top_k < 16 * wl.shape.n_experts for n in sizes]
        n_small = sum(dc and n <= 192 for n, dc in zip(sizes, decode))
        # decode-tile chunks of 193 to 512 tokens run their shared gate/up inside their gate/up
        # launch and leave their shared down + combine to the next one (in this layer call)
        n_defer = sum(dc and 192 < n <= 512 for n, dc in zip(sizes, decode))
        assert 0 < n_small
        assert prof["gu_mixed"][1] == n_small + n_defer and prof["down_mixed"][1] == n_small
        assert prof["combine"][1] == n_small and prof["down_shared"][1] == 0
        assert prof["down_shared_combine"][1] == len(sizes) - n_small
        assert prof["gu_shared"][1] == len(sizes) - n_small - n_defer
        assert torch.equal(bits(got["out"]), bits(base["out"])), chunk


@pytest.mark.parametrize("T,chunk", [(600, 128), (40, 8)])
def test_graph_capture_resident_layer(moe, T, chunk):
    """With every expert resident a layer call enqueues kernels only (no allocation, host
    synchronisation or memset), so the whole call (route + 5 chunks) can be captured in a HIP
    graph (chunks of 128 tokens, and of 8, whose shared expert runs inside the routed
    launches). Replays, with eager work and synchronisation between them, give the eager bytes
    every time."""
    wl = mi.custom_workload("graph", T=T, d=256, E=32, k=4, inter=128, inter_shared=256,
                            zipf_s=1.1, seed=17)
    params, L = place(wl)
    x = mi.make_x(wl, device="cuda")
    eager = _run(moe, L, x, chunk)
    bufs = moe.layer_buffers(L, wl.T, chunk)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                      # warm-up outside the capture
        moe.moe_prefill_layer(L, x, chunk, bufs=bufs)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.moe_prefill_layer(L, x, chunk, bufs=bufs)
    for _ in range(3):
        for key in ("out", "logits"):
            bufs[key].zero_()
        bufs["ids"].fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(bits(bufs["out"]), bits(eager["out"]))
        assert torch.equal(bufs["ids"], eager["ids"])
        assert torch.equal(bufs["chunk_counts"], eager["chunk_counts"])
