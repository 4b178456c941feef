#!/usr/bin/env python3
"""Benchmark of expert-major deep prefill of one routed MoE layer on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1]

Workload (headline): one layer with d = 2048, E = 512 routed experts, top-8, expert
intermediate 512 and a shared expert of intermediate 2048, bf16 storage with fp32
accumulation, T = 16,022 prompt tokens routed without bias, all experts resident in HBM, run
as the batched pass (one chunk of T rows). Inputs and weights are seeded synthetic tensors,
already in HBM when timing starts. One step = the whole path once: router GEMM, top-k,
per-chunk counts, bucketing (histogram, scan, permute), shared and routed grouped GEMMs with
the fused SiLU epilogue, and the combine (folded into the shared down GEMM's epilogue).

Prints one JSON line (stdout). Per-kernel times come from HIP events that the library records
around each of its launches on the launch's own stream, over a second pass of the same K
steps (the headline time comes from a pass without those events). Also reported: the same
layer at deep chunks 2,048 / 4,096 / 8,192, the layer with all experts streamed from a pinned
host bank through a 64-line ring at chunk 2,048 (with the measured host-link rate and the
share of compute hidden under the copies), a decode-sized call (8 tokens) eager and as a
replayed HIP graph, an 8-layer stack (T = 32,700, Zipf routing, half
the experts through one 128-line ring), and the fp64 CPU oracle on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer prefill tokens/s and MFMA TFLOP/s fraction at T=16k, E=512, k=8"
PEAK_BF16 = 2.5e15      # dense bf16 MFMA, FLOP/s
PEAK_HBM = 8.0e12       # HBM3E, B/s


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic(stage: str, T: int, sh, counts):
    """(flops, bytes) of one step's launches of a stage: data each kernel must touch once
    (weights of used experts, activations, intermediates, outputs), no padding."""
    d, E, k, I, Is = sh.d, sh.n_experts, sh.top_k, sh.inter, sh.inter_shared
    Ns = T * k
    used = int((counts > 0).sum())
    if stage == "router":
        return 2 * T * d * E, T * d * 2 + E * d * 2 + T * E * 4
    if stage == "topk":
        return 0, T * E * 4 + T * k * 8
    if stage == "gu_routed":
        # each prompt row is read once (its reads for its other k - 1 experts are re-reads,
        # not algorithmic bytes), the used experts' gate/up weights once, h written once
        return 2 * Ns * d * 2 * I, used * 2 * I * d * 2 + T * d * 2 + Ns * I * 2
    if stage == "gu_mixed":                # both gate/up GEMMs in one launch; x read once
        f1, b1 = algorithmic("gu_routed", T, sh, counts)
        f2, b2 = algorithmic("gu_shared", T, sh, counts)
        return f1 + f2, b1 + b2 - T * d * 2
    if stage == "down_routed":
        return 2 * Ns * I * d, used * d * I * 2 + Ns * I * 2 + Ns * d * 4
    if stage == "gu_shared":
        return 2 * T * d * 2 * Is, 2 * Is * d * 2 + T * d * 2 + T * Is * 2
    if stage == "down_shared":
        return 2 * T * Is * d, d * Is * 2 + T * Is * 2 + T * d * 4
    if stage == "combine":
        return 2 * Ns * d, Ns * d * 4 + T * d * 4 + T * k * 4 + T * d * 2
    if stage == "down_shared_combine":     # shared down GEMM with the combine in its epilogue
        return (2 * T * Is * d + 2 * Ns * d,
                d * Is * 2 + T * Is * 2 + Ns * d * 4 + T * k * 4 + T * d * 2)
    if stage in ("hist", "permute"):
        return 0, Ns * 4 * (1 if stage == "hist" else 3)
    return 0, 0


def _shape(wl):
    import routed_expert_grouped_moe_amd as moe
    s = wl.shape
    return moe.make_shape(s.d, s.n_experts, s.top_k, s.inter, s.inter_shared, s.dtype)


def _place(wl, layer=0, offloaded=(), ring=None, params=None):
    """(params on cuda:0, library Layer) for one layer of a workload."""
    import moe_inputs as mi
    import routed_expert_grouped_moe_amd as moe
    if params is None:
        params = mi.make_layer(wl, layer, device="cuda")
    return params, moe.Layer.from_params(params, _shape(wl), "cuda", offloaded, ring, layer)


def time_steps(fn, steps, warmup, gate=False):
    """(mean ms per step over the K steps, wall ms per step, per-step ms list). HIP events on
    the current stream bracket the K steps, and each step separately. gate: the GPU first
    spins for about 50 ms while the host enqueues the K steps behind it, so no kernel of the
    timed steps waits on the host (per-launch event timings then hold kernel time only)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    w0 = time.perf_counter()
    if gate:
        torch.cuda._sleep(100_000_000)
    ev[0].record()
    for i in range(steps):
        fn()
        ev[i + 1].record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - w0) * 1e3 / steps
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    return ev[0].elapsed_time(ev[steps]) / steps, wall, per


def spread(per):
    import numpy as np
    a = np.asarray(per)
    return {"median": round(float(np.median(a)), 4), "min": round(float(a.min()), 4),
            "max": round(float(a.max()), 4)}


def h2d_probe(nbytes: int, runs: int) -> float:
    """Pinned host -> HBM copy rate (GB/s) of one nbytes transfer on a side stream."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()
    best = float("inf")
    for _ in range(runs):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        with torch.cuda.stream(s):
            dst.copy_(src, non_blocking=True)
        s.synchronize()
        best = min(best, time.perf_counter() - t0)
    return nbytes / best / 1e9


def small_call_variant(L, mi, wl, T: int = 8, steps: int = 50):
    """A decode-sized call (T tokens of the headline layer, one chunk) eager and as a
    replayed HIP graph of the same call: at this size launch overhead, not the GPU, bounds
    the eager call."""
    import torch

    import routed_expert_grouped_moe_amd as moe
    x = mi.make_x(wl, device="cuda")[:T].contiguous()
    bufs = moe.layer_buffers(L, T, T)
    call = lambda: moe.moe_prefill_layer(L, x, T, bufs=bufs)
    e_ms, e_wall, _ = time_steps(call, steps, 5)
    ref = bufs["out"].clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    g_ms, g_wall, _ = time_steps(g.replay, steps, 5)
    ok = torch.equal(bufs["out"].view(torch.int16), ref.view(torch.int16))
    # the same calls enqueued behind a GPU spin: the GPU's own time per call, without the
    # host's launch work between calls
    eg_ms, _, _ = time_steps(call, steps, 0, gate=True)
    gg_ms, _, _ = time_steps(g.replay, steps, 0, gate=True)
    return {"tokens": T, "eager_ms_per_call": round(e_wall, 4),
            "graph_ms_per_call": round(g_wall, 4),
            "eager_gpu_ms": round(e_ms, 4), "graph_gpu_ms": round(g_ms, 4),
            "eager_gpu_ms_host_ahead": round(eg_ms, 4),
            "graph_gpu_ms_host_ahead": round(gg_ms, 4),
            "graph_equals_eager": bool(ok)}


def stack_variant(steps: int):
    """The 8-layer stack (T = 32,700, Zipf(1.5) routing, RMSNorm + residual between layers,
    experts 256..511 of every layer in pinned banks streamed through one 128-line ring,
    chunk 2,048): one untimed pass, then `steps` timed passes."""
    import torch

    import moe_inputs as mi
    import routed_expert_grouped_moe_amd as moe
    wl = mi.WORKLOADS["stack_32700"]
    E = wl.shape.n_experts
    off = range(E - wl.n_offloaded, E)
    ring, layers = moe.Ring(_shape(wl), wl.ring_lines), []
    for layer in range(wl.n_layers):
        p = mi.make_layer(wl, layer, device="cuda")
        layers.append(_place(wl, layer=layer, offloaded=off, ring=ring, params=p)[1])
        del p
    x = mi.make_x(wl, device="cuda")
    cs = torch.cuda.Stream()
    run = lambda: moe.moe_prefill_stack(layers, x, 2048, wl.rmsnorm_eps, copy_stream=cs)
    run()
    torch.cuda.synchronize()
    ring.reset_stats()
    _, wall, per = time_steps(run, steps, 0)
    st = ring.stats()
    ring.close()
    looks = st["hits"] + st["misses"] + st["pinned_uses"]
    return {"workload": f"stack_{wl.n_layers}x_T{wl.T}_zipf1.5_ring{wl.ring_lines}_chunk2048",
            "tokens_per_s": round(wl.T / (wall / 1e3), 1), "ms_per_pass": round(wall, 1),
            "pass_ms": spread(per),
            # experts served without a copy: staged hits and uses of lines pinned for a layer
            "ring_hit_rate": round((st["hits"] + st["pinned_uses"]) / max(1, looks), 4),
            "pinned_uses_per_pass": st["pinned_uses"] // steps,
            "ring_lookups_per_pass": looks // steps,
            "h2d_gb_per_pass": round(st["bytes_h2d"] / steps / 1e9, 2),
            "h2d_gb_per_pass_by_kind": {k: round(v / steps / 1e9, 3)
                                        for k, v in st["copied_bytes"].items()},
            "requested_gb_per_pass_by_kind": {k: round(v / steps / 1e9, 3)
                                              for k, v in st["requested_bytes"].items()},
            "h2d_gbps": round(st["bytes_h2d"] / steps / (wall / 1e3) / 1e9, 2)}


def fused_variant(moe, L, x, bufs, T, steps):
    """The layer at chunks whose routed tiles are 64 rows (1,024 and 2,048 tokens: 16 and 32
    rows per expert) with the routed GEMMs as two launches and as the fused launch
    (MOE_OPT_FUSED_GU_DOWN, h kept in LDS): layer time, routed-GEMM time per layer from the
    library's launch timings, and bit-identity with the batched pass."""
    import torch
    res = {}
    for c in (1024, 2048):
        b2 = moe.layer_buffers(L, T, c)
        ent = {}
        for name, on in (("separate", 0), ("fused", 1)):
            moe.moe_set_option("fused_gu_down", on)
            try:
                run = lambda: moe.moe_prefill_layer(L, x, c, bufs=b2)
                v_ms, _, v_per = time_steps(run, max(3, steps // 2), 2)
                moe.moe_profile_read(reset=True)
                moe.moe_profile_enable(True)
                time_steps(run, 3, 0, gate=True)
                moe.moe_profile_enable(False)
                prof = moe.moe_profile_read(reset=True)
            finally:
                moe.moe_set_option("fused_gu_down", 0)
                moe.moe_profile_enable(False)
            # every GEMM stage (the separate path runs the routed gate/up inside the mixed
            # launch with the shared expert's, the fused one runs the shared gate/up alone)
            gemm = sum(prof[s][0] for s in ("gu_routed", "down_routed", "gu_down_fused",
                                             "gu_mixed", "gu_shared", "down_shared_combine")) / 3
            ok = torch.equal(b2["out"].view(torch.int16), bufs["out"].view(torch.int16))
            ent[name] = {"ms_per_step": round(v_ms, 3), "step_ms": spread(v_per),
                         "gemm_ms_per_step": round(gemm, 3),
                         "stage_ms_per_step": {k: round(v[0] / 3, 3) for k, v in prof.items()
                                               if v[1]},
                         "fused_launches_per_step": prof["gu_down_fused"][1] // 3,
                         "bit_identical_to_batched": bool(ok)}
        res[f"chunk{c}"] = ent
        del b2
    return res


def ring_variant(moe, wl, params, x, bufs, t_gemm):
    """The layer as the config specifies it: all 512 experts in a pinned bank, streamed
    through a 64-line ring at chunk 2,048 (one untimed pass, three timed). t_gemm: the same
    layer's resident time at chunk 2,048 (ms), the compute alone."""
    import torch
    T = wl.T
    log("[bench] ring variant: all 512 experts in a pinned bank, 64 lines, chunk 2048")
    sh = _shape(wl)
    ring = moe.Ring(sh, 64)
    _, Lr = _place(wl, offloaded=range(sh.n_experts), ring=ring, params=params)
    br = moe.layer_buffers(Lr, T, 2048)
    cs = torch.cuda.Stream()
    ring_step = lambda: moe.moe_prefill_layer(Lr, x, 2048, bufs=br, copy_stream=cs)
    ring_step()
    torch.cuda.synchronize()
    ring.reset_stats()
    r_ms, r_wall, r_per = time_steps(ring_step, 3, 0)
    ok = torch.equal(br["out"].view(torch.int16), bufs["out"].view(torch.int16))
    st = ring.stats()
    per_step_bytes = st["bytes_h2d"] / 3
    link = h2d_probe(1 << 30, 3)
    line_rate = h2d_line_probe(ring.line_bytes, 64)
    # the copies at the link rate of one 1 GiB pinned copy: a floor the 6 MiB line copies of
    # the ring do not reach, so the compute share below is a lower bound
    t_copy = per_step_bytes / (link * 1e9) * 1e3
    # the same bytes as 6 MiB line copies alternating two streams with nothing else on the
    # GPU (the ring's copy pattern): the copy time the ring would take without compute
    t_lines = per_step_bytes / (line_rate * 1e9) * 1e3
    hidden = (t_copy + t_gemm - r_wall) / t_gemm
    hidden_lines = (t_lines + t_gemm - r_wall) / t_gemm
    res = {
        "tokens_per_s": round(T / (r_wall / 1e3), 1), "ms_per_step": round(r_wall, 2),
        "step_ms": spread(r_per),
        "h2d_gb_per_step": round(per_step_bytes / 1e9, 3),
        "h2d_gbps": round(per_step_bytes / (r_wall / 1e3) / 1e9, 2),
        "h2d_link_gbps_measured": round(link, 2),
        "link_floor_ms": round(t_copy, 2),
        "ring_over_link_floor": round(r_wall / t_copy, 4),
        "compute_alone_ms": t_gemm,
        "ring_hit_rate": round((st["hits"] + st["pinned_uses"]) /
                               max(1, st["hits"] + st["misses"] + st["pinned_uses"]), 4),
        "copy_waits_per_step": st["copy_waits"] // 3,
        "copied_bytes_per_step_by_kind": {k: v // 3 for k, v in st["copied_bytes"].items()},
        "compute_hidden_frac_vs_link_floor": round(max(0.0, min(1.0, hidden)), 3),
        "h2d_line_copy_gbps_measured": round(line_rate, 2),
        "line_copies_alone_ms": round(t_lines, 2),
        "compute_hidden_frac_vs_line_copies": round(max(0.0, min(1.0, hidden_lines)), 3),
        "bit_identical_to_batched": bool(ok)}
    del br, Lr
    ring.close()
    return res


def _union(iv):
    out = []
    for a, b in sorted(iv):
        if out and a <= out[-1][1]:
            out[-1][1] = max(out[-1][1], b)
        else:
            out.append([a, b])
    return out


def _cover(u):
    return sum(b - a for a, b in u)


def _meet(u, v):
    """Length of the intersection of two interval unions (each sorted and disjoint)."""
    i = j = 0
    tot = 0
    while i < len(u) and j < len(v):
        lo, hi = max(u[i][0], v[j][0]), min(u[i][1], v[j][1])
        tot += max(0, hi - lo)
        if u[i][1] < v[j][1]:
            i += 1
        else:
            j += 1
    return tot


def overlap_from_trace(d: str) -> dict:
    """Copy/compute overlap of the ring passes in a rocprofv3 trace of a bench.py run
    (`rocprofv3 --kernel-trace --memory-copy-trace --output-format csv`).

    Copies are the library's line-copy kernels when the run has any (the all-offloaded ring
    layer), else the host-to-device DMA copies; the window runs from the first copy after the
    first router launch to the end of the last copy, so it covers the ring passes of a run
    with `--variants ring` or `--variants stack` and nothing of the input set-up. Inside it: the share of time some copy is in flight, and the share
    of the GEMM kernels' busy time (and of all library kernels' busy time) that runs while a
    copy is in flight, measured from the timeline rather than bounded from separate runs."""
    import csv
    import glob
    kt = sorted(glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True))
    mt = sorted(glob.glob(os.path.join(d, "**", "*memory_copy_trace.csv"), recursive=True))
    if not kt:
        raise SystemExit(f"no *kernel_trace.csv under {d}")
    kernels = []
    for path in kt:
        for r in csv.DictReader(open(path)):
            kernels.append((r["Kernel_Name"], int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    copies = []
    for path in mt:
        for r in csv.DictReader(open(path)):
            if any("HOST_TO_DEVICE" in str(v) for v in r.values()):
                copies.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    lib = [k for k in kernels if "moe::" in k[0]]
    kcopies = [(a, b) for n, a, b in lib if "line_copy_kernel" in n]
    if kcopies:     # a ring run whose copies are kernels; DMA copies are the later link probes
        copies = kcopies
    first_router = min((a for n, a, b in lib if "router_kernel" in n), default=None)
    if first_router is None or not copies:
        return {"trace": d, "error": "no router launch or no host-to-device copies in the trace"}
    copies = [c for c in copies if c[0] >= first_router]
    if not copies:
        return {"trace": d, "error": "no copies after the first router launch"}
    w0, w1 = min(a for a, _ in copies), max(b for _, b in copies)
    inside = lambda a, b: a >= w0 and b <= w1
    cu = _union(copies)
    comp = [k for k in lib if "line_copy_kernel" not in k[0] and inside(k[1], k[2])]
    gemm = _union([(a, b) for n, a, b in comp if "gu_" in n or "down_kernel" in n])
    allk = _union([(a, b) for _, a, b in comp])
    win = w1 - w0
    res = {"trace": d, "window_ms": round(win / 1e6, 3), "copies": len(copies),
           "link_busy_frac": round(_cover(cu) / win, 4),
           "gemm_busy_ms": round(_cover(gemm) / 1e6, 3),
           "gemm_under_copy_frac": round(_meet(gemm, cu) / max(1, _cover(gemm)), 4),
           "kernels_busy_ms": round(_cover(allk) / 1e6, 3),
           "kernels_under_copy_frac": round(_meet(allk, cu) / max(1, _cover(allk)), 4),
           "copy_kind": "kernel" if kcopies else "dma"}
    return res


def kernel_source_sha() -> str:
    import hashlib
    p = os.path.join(ROOT, "routed_expert_grouped_moe_amd", "csrc", "gemm.hip")
    with open(p, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summary, or None when the
    summary is missing or was taken on a different kernel source."""
    p = os.path.join(ROOT, "profiles", "hbm_traffic_T16022_batched.md")
    if not os.path.exists(p):
        return None
    text = open(p).read()
    start = text.find("```json")
    if start < 0:
        return None
    blob = json.loads(text[start + 7: text.find("```", start + 7)])
    if blob.get("source_sha256") != kernel_source_sha():
        return None
    k = blob.get("kernels", {}).get(kernel)
    return None if k is None else int(k["traffic_bytes_per_launch"])


def copy_probe(nbytes: int, runs: int) -> float:
    """A plain copy kernel: out = in * 1 over nbytes of fp32 (reads and writes nbytes each)."""
    import torch
    a = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    ms, _, _ = time_steps(lambda: torch.mul(a, 1.0, out=b), runs, 1)
    return 2 * a.numel() * 4 / (ms / 1e3) / 1e9


def cpu_baseline(params, wl, x, seconds, chunk=1024):
    """The fp64 oracle on the first tokens of the workload, in whole chunks of `chunk` tokens
    until about `seconds` of CPU work have run (the rate differs a lot between hosts)."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import moe_inputs as mi
    import oracle.moe_oracle as orc
    from tests.parity import oracle_params
    op = oracle_params(params, wl)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    done, dt = 0, 0.0
    while done < wl.T and dt < seconds:
        n = min(chunk, wl.T - done)
        xs = mi.to_numpy_exact(x[done:done + n])
        t0 = time.perf_counter()
        orc.moe_layer(xs, op)
        dt += time.perf_counter() - t0
        done += n
    sh = wl.shape
    flop = done * (2 * sh.d * sh.n_experts + 6 * sh.d * sh.inter * sh.top_k
                   + 6 * sh.d * sh.inter_shared)
    return {"value": round(done / dt, 2), "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"first {done} of the {wl.T} tokens in chunks of {chunk}, same layer "
                      f"(all 512 experts widened from bf16 as used), fp64 numpy, {dt:.1f} s",
            "gflops_fp64": round(flop / dt / 1e9, 2)}


def cpu_baseline_configs(sample_tokens=256):
    """The fp64 oracle on the first tokens of the three smaller workloads (the tiny fp32
    layer, the 3,001-token layer and the 4,099-token chunk-gate layer), once on one BLAS
    thread and once on all of them."""
    from threadpoolctl import threadpool_info, threadpool_limits

    import moe_inputs as mi
    import oracle.moe_oracle as orc
    from tests.parity import oracle_params
    res = {}
    for name in ("tiny_fp32", "layer_3001", "chunk_gate_4099"):
        wl = mi.WORKLOADS[name]
        params = mi.make_layer(wl, device="cuda")
        n = min(wl.T, sample_tokens)
        xs = mi.to_numpy_exact(mi.make_x(wl, device="cuda", T=n))
        op = oracle_params(params, wl)
        del params
        ent = {"tokens": n}
        for label, lim in (("one_core", 1), ("all_cores", None)):
            with threadpool_limits(limits=lim):
                threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
                t0 = time.perf_counter()
                orc.moe_layer(xs, op)
                dt = time.perf_counter() - t0
            ent[label] = {"tokens_per_s": round(n / dt, 2), "cores": int(threads),
                          "seconds": round(dt, 2)}
        res[name] = ent
        del op
    return res


def h2d_line_probe(line_bytes: int, n_lines: int, runs: int = 2) -> float:
    """Pinned host -> HBM rate (GB/s) of n_lines copies of one expert line each, alternating
    two streams as the ring's copies do."""
    import torch
    src = torch.empty(n_lines * line_bytes, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(n_lines * line_bytes, dtype=torch.uint8, device="cuda")
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    best = float("inf")
    for _ in range(runs):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(n_lines):
            with torch.cuda.stream(streams[i % 2]):
                dst[i * line_bytes:(i + 1) * line_bytes].copy_(
                    src[i * line_bytes:(i + 1) * line_bytes], non_blocking=True)
        for s in streams:
            s.synchronize()
        best = min(best, time.perf_counter() - t0)
    return n_lines * line_bytes / best / 1e9


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-sample-seconds", type=float, default=12.0,
                    help="seconds of fp64 oracle work on the headline workload's first tokens "
                         "(whole chunks of 1,024 tokens)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-variants", action="store_true")
    ap.add_argument("--no-stack", action="store_true",
                    help="skip the 8-layer T=32,700 stack variant (about a minute)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run a plain fp32 copy kernel (out = in * 1) over BYTES bytes "
                         "5 times and print its bandwidth (calibrates HBM byte counters)")
    ap.add_argument("--variants", default="chunks,small,fused,ring,stack",
                    help="comma list of the variants to run beside the headline pass "
                         "(chunks, small, fused, ring, stack)")
    ap.add_argument("--overlap-from-trace", metavar="DIR", default="",
                    help="no GPU work: read a rocprofv3 kernel and memory-copy trace (csv) of a "
                         "bench.py run from DIR and print the copy/compute overlap of its ring "
                         "passes")
    args = ap.parse_args()
    if args.overlap_from_trace:
        print(json.dumps(overlap_from_trace(args.overlap_from_trace)), flush=True)
        return
    chosen = set() if args.no_variants else {v for v in args.variants.split(",") if v}
    if args.no_stack:
        chosen.discard("stack")
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        log("bench.py runs on one GPU only: the library has no multi-GPU path "
            "(no collectives or sharding); run it with --gpus 1.")
        sys.exit(2)

    import numpy as np
    import torch

    import moe_inputs as mi
    import routed_expert_grouped_moe_amd as moe

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.copy_probe:
        gbps = copy_probe(args.copy_probe, 5)
        print(json.dumps({"copy_probe_bytes": args.copy_probe, "runs": 5,
                          "read_plus_write_gbps": round(gbps, 1)}), flush=True)
        return
    # The stack variant runs first, in a fresh process state: after the other variants its
    # host-link rate measured about 15% lower (1.57 s against 1.35 s per pass) while alone,
    # or after any one of them, it holds 52-53 GB/s.
    stack = None
    if "stack" in chosen:
        log("[bench] stack variant: 8 layers, T=32,700, 128-line ring")
        stack = stack_variant(1)
        torch.cuda.empty_cache()
    wl = mi.WORKLOADS["offload_16022"]      # T = 16,022 inputs (seeded), placed resident here
    T = wl.T
    log(f"[bench] generating layer and {T} tokens on cuda:0")
    params, L = _place(wl)
    x = mi.make_x(wl, device="cuda")
    sh = L.shape
    torch.cuda.synchronize()

    bufs = moe.layer_buffers(L, T, T)
    step = lambda: moe.moe_prefill_layer(L, x, T, bufs=bufs)
    log(f"[bench] batched pass: warmup {args.warmup}, steps {args.steps}")
    ms, wall_ms, per_step = time_steps(step, args.steps, args.warmup)
    counts = bufs["chunk_counts"][0].cpu().numpy()

    moe.moe_profile_read(reset=True)
    moe.moe_profile_enable(True)
    ms_prof, _, _ = time_steps(step, args.steps, 0, gate=True)
    moe.moe_profile_enable(False)
    prof3 = moe.moe_profile_read(reset=True, clocks=True)
    prof = {k: (v[0], v[1]) for k, v in prof3.items()}

    flop_tok = 2 * sh.d * sh.n_experts + 6 * sh.d * sh.inter * sh.top_k + 6 * sh.d * sh.inter_shared
    tok_s = T / (ms / 1e3)
    tflops = flop_tok * T / (ms / 1e3) / 1e12
    kernels = {}
    for stage, (tot_ms, n) in prof.items():
        if n == 0:
            continue
        per_launch_ms = tot_ms / n
        f, b = algorithmic(stage, T, sh, counts)
        per_step_launches = n / args.steps
        f_l, b_l = f / per_step_launches, b / per_step_launches
        ent = {"ms_per_step": round(tot_ms / args.steps, 4), "launches_per_step": per_step_launches,
               "avg_launch_us": round(per_launch_ms * 1e3, 2)}
        if f:
            ent["tflops"] = round(f_l / (per_launch_ms / 1e3) / 1e12, 2)
            ent["mfma_frac"] = round(ent["tflops"] * 1e12 / PEAK_BF16, 4)
        if b:
            ent["gbps"] = round(b_l / (per_launch_ms / 1e3) / 1e9, 1)
            ent["hbm_frac"] = round(ent["gbps"] * 1e9 / PEAK_HBM, 4)
            tr = measured_traffic(stage)
            if tr is not None:
                # HBM bytes the counters saw over the algorithmic bytes: re-reads and waste
                ent["traffic_over_algorithmic"] = round(tr / b_l, 3)
        if prof3[stage][2] > 0:
            ent["clock_mhz"] = round(prof3[stage][2], 0)
        kernels[stage] = ent
    gemm = [s for s in ("gu_mixed", "gu_routed", "down_routed", "gu_shared", "down_shared",
                        "down_shared_combine") if prof[s][1] > 0]
    gemm_ms = sum(prof[s][0] for s in gemm) / args.steps
    # GEMM flops only (the fused combine's 2*k*d per token is not matrix work)
    gemm_flop = sum(algorithmic(s, T, sh, counts)[0] for s in gemm) - (
        2 * T * sh.top_k * sh.d if "down_shared_combine" in gemm else 0)
    dom = max(gemm, key=lambda s: prof[s][0])
    f, b = algorithmic(dom, T, sh, counts)
    n_l = prof[dom][1] / args.steps
    avg_s = prof[dom][0] / prof[dom][1] / 1e3
    t_mfma, t_hbm = (f / n_l) / PEAK_BF16, (b / n_l) / PEAK_HBM
    if t_hbm >= t_mfma:
        ach = (b / n_l) / avg_s / 1e9
        roof = {"kernel": dom, "bound": "hbm", "achieved": round(ach, 1), "peak": 8000.0,
                "unit": "GB/s", "frac": round(ach / 8000.0, 4), "traffic": measured_traffic(dom),
                "bytes_per_launch": int(b / n_l), "avg_launch_us": round(avg_s * 1e6, 2),
                "flops_per_launch": int(f / n_l),
                "mfma_frac": round((f / n_l) / avg_s / PEAK_BF16, 4)}
    else:
        ach = (f / n_l) / avg_s / 1e12
        roof = {"kernel": dom, "bound": "mfma", "achieved": round(ach, 1), "peak": 2500.0,
                "unit": "TFLOP/s", "frac": round(ach / 2500.0, 4), "traffic": measured_traffic(dom),
                "flops_per_launch": int(f / n_l), "avg_launch_us": round(avg_s * 1e6, 2)}
    if roof["traffic"] is not None:
        roof["traffic_over_algorithmic"] = round(roof["traffic"] / (b / n_l), 3)
    clk = prof3[dom][2]
    if clk > 0:
        # the shader clock the kernel ran at (sampled in the kernel): the MFMA peak scales with
        # it (2.5 PFLOP/s is quoted at 2.4 GHz)
        roof["clock_mhz_sustained"] = round(clk, 0)
        roof["mfma_peak_at_sustained_clock_tflops"] = round(2500.0 * clk / 2400.0, 1)

    variants = {}
    for c in ((2048, 4096, 8192) if "chunks" in chosen else ()):
        b2 = moe.layer_buffers(L, T, c)
        v_ms, _, v_per = time_steps(lambda: moe.moe_prefill_layer(L, x, c, bufs=b2),
                                    max(3, args.steps // 2), 2)
        ok = torch.equal(b2["out"].view(torch.int16), bufs["out"].view(torch.int16))
        variants[f"resident_chunk{c}"] = {"tokens_per_s": round(T / (v_ms / 1e3), 1),
                                          "ms_per_step": round(v_ms, 3), "step_ms": spread(v_per),
                                          "bit_identical_to_batched": bool(ok)}
        del b2
    if "small" in chosen:
        variants["small_call_T8"] = small_call_variant(L, mi, wl)
    if "fused" in chosen:
        variants["fused_gu_down"] = fused_variant(moe, L, x, bufs, T, args.steps)
    if "ring" in chosen:
        if "resident_chunk2048" in variants:
            t_gemm = variants["resident_chunk2048"]["ms_per_step"]    # ms, compute alone
        else:
            b2 = moe.layer_buffers(L, T, 2048)
            t_gemm = round(time_steps(lambda: moe.moe_prefill_layer(L, x, 2048, bufs=b2), 3, 2)[0], 3)
            del b2
        variants["offload_ring64_chunk2048"] = ring_variant(moe, wl, params, x, bufs, t_gemm)
    if stack is not None:
        variants["stack"] = stack

    copy_gbps = copy_probe(1 << 30, 5)
    cpu = None
    if not args.no_cpu_baseline:
        log(f"[bench] CPU oracle baseline, about {args.cpu_sample_seconds:.0f} s")
        cpu = cpu_baseline(params, wl, x, args.cpu_sample_seconds)
        del params, L, bufs
        torch.cuda.empty_cache()
        log("[bench] CPU oracle on the three smaller workloads, one core and all cores")
        cpu["other_workloads"] = cpu_baseline_configs()

    line = {
        "metric": METRIC, "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "step_ms": spread(per_step),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: seeded Gaussian activations and random-init weights "
                "(1/sqrt(fan_in)), router std 0.02, uniform routing",
        "config": {"workload": "moe_layer_T16022_d2048_E512_k8_I512_shared2048_resident_batched",
                   "T": T, "chunk": T, "d": sh.d, "n_experts": sh.n_experts, "top_k": sh.top_k,
                   "inter": sh.inter, "inter_shared": sh.inter_shared, "experts": "resident"},
        "tflops": round(tflops, 2), "mfma_frac": round(tflops * 1e12 / PEAK_BF16, 4),
        "grouped_gemm_mfma_frac": round(gemm_flop / (gemm_ms / 1e3) / PEAK_BF16, 4),
        "wall_ms_per_step": round(wall_ms, 4), "ms_per_step_profiled": round(ms_prof, 4),
        "hbm_copy_gbps_measured": round(copy_gbps, 1),
        "roofline": roof, "cpu_baseline": cpu, "kernels": kernels, "variants": variants,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
