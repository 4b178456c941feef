"""MI355X (gfx950) expert-major "deep" prefill of a routed mixture-of-experts layer.

Thin Python binding of libmoeprefill (include/moe_prefill.h): the functions below carry the C
names and only marshal arguments (torch tensors -> device pointers, the current HIP stream ->
a raw handle). Every step of the computation runs in the library's HIP kernels; PyTorch is
used for device memory, pinned host memory and streams. There is no CPU fallback: without
the built library every call raises.
"""
from __future__ import annotations

import ctypes
from typing import Iterable, Optional, Sequence

import torch

from ._abi import (MOE_BF16, MOE_F32, MoeError, MoeLayer, MoeRingStats, MoeShape, MoeWsOffsets,
                   check, lib)

__all__ = [
    "MOE_BF16", "MOE_F32", "MoeError", "Layer", "Ring", "make_shape", "moe_workspace_bytes",
    "moe_layer_workspace_bytes",
    "moe_prefill_route", "moe_prefill_chunk", "moe_prefill_layer", "moe_stage_experts",
    "moe_add_rmsnorm", "moe_abi_version", "line_elems", "moe_workspace_offsets",
    "layer_buffers", "moe_profile_enable", "moe_profile_read", "moe_prefill_stack",
    "moe_set_option", "moe_get_option",
]


def _vp(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(s: Optional[torch.cuda.Stream] = None):
    s = s if s is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _torch_dtype(dtype: int):
    return torch.bfloat16 if dtype == MOE_BF16 else torch.float32


def _need(t: torch.Tensor, name: str, dtype, shape=None):
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")


def moe_abi_version() -> int:
    return lib().moe_abi_version()


def make_shape(d, n_experts, top_k, inter, inter_shared, dtype="bf16") -> MoeShape:
    dt = MOE_BF16 if dtype in ("bf16", MOE_BF16, torch.bfloat16) else MOE_F32
    return MoeShape(d, n_experts, top_k, inter, inter_shared, dt)


def line_elems(sh: MoeShape) -> int:
    """Elements of one expert line: W_gu [2I, d] then W_down [d, I]."""
    return 3 * sh.inter * sh.d


def moe_workspace_bytes(sh: MoeShape, max_chunk_tokens: int) -> int:
    return int(lib().moe_workspace_bytes(ctypes.byref(sh), int(max_chunk_tokens)))


def moe_layer_workspace_bytes(sh: MoeShape, T: int, chunk: int) -> int:
    return int(lib().moe_layer_workspace_bytes(ctypes.byref(sh), int(T), int(chunk)))


def moe_workspace_offsets(sh: MoeShape, n: int) -> dict:
    """Byte offsets of a chunk call's member lists inside its workspace (n rows)."""
    o = MoeWsOffsets()
    check(lib().moe_workspace_offsets(ctypes.byref(sh), int(n), ctypes.byref(o)),
          "moe_workspace_offsets")
    return {f: getattr(o, f) for f, _ in MoeWsOffsets._fields_}


class Ring:
    """A ring of `n_lines` device expert lines (moe_ring), its device memory and banks."""

    def __init__(self, sh: MoeShape, n_lines: int, device="cuda"):
        self.shape = sh
        self.n_lines = int(n_lines)
        esz = 2 if sh.dtype == MOE_BF16 else 4
        self.line_bytes = line_elems(sh) * esz
        self.lines = torch.empty(self.n_lines * self.line_bytes, dtype=torch.uint8, device=device)
        h = ctypes.c_void_p()
        check(lib().moe_ring_create(ctypes.byref(sh), _vp(self.lines), self.n_lines,
                                    ctypes.byref(h)), "moe_ring_create")
        self.handle = h
        self._banks = {}

    def bind_bank(self, layer_id: int, bank: torch.Tensor, slot_of_expert: Sequence[int]):
        """bank: pinned host tensor [slots, line_elems]; slot_of_expert[e] = row or -1."""
        if bank.numel() and not bank.is_pinned():
            raise ValueError("bank must be pinned host memory")
        E = self.shape.n_experts
        if len(slot_of_expert) != E:
            raise ValueError("slot_of_expert needs one entry per expert")
        slots = (ctypes.c_int32 * E)(*[int(v) for v in slot_of_expert])
        check(lib().moe_ring_bind_bank(self.handle, int(layer_id),
                                       _vp(bank) if bank.numel() else None, slots),
              "moe_ring_bind_bank")
        self._banks[int(layer_id)] = bank

    def stats(self) -> dict:
        """Ring counters; requested_bytes / copied_bytes are dicts by kind of staging
        (initial, ahead, demand, cross_layer)."""
        from ._abi import COPY_KINDS
        st = MoeRingStats()
        check(lib().moe_ring_stats(self.handle, ctypes.byref(st)), "moe_ring_stats")
        out = {}
        for f, _ in MoeRingStats._fields_:
            v = getattr(st, f)
            out[f] = {k: int(v[i]) for i, k in enumerate(COPY_KINDS)} if f.endswith("_bytes") else v
        return out

    def prefetch(self, layer_id: int, experts: Sequence[int], copy_stream=None):
        """moe_ring_prefetch: stage experts of a later layer without holding their lines."""
        n = len(experts)
        ex = (ctypes.c_int32 * max(n, 1))(*[int(e) for e in experts])
        check(lib().moe_ring_prefetch(self.handle, int(layer_id), ex, n, _stream(copy_stream)),
              "moe_ring_prefetch")

    def reset_stats(self):
        check(lib().moe_ring_reset_stats(self.handle), "moe_ring_reset_stats")

    def invalidate(self):
        check(lib().moe_ring_invalidate(self.handle), "moe_ring_invalidate")

    def line_ptr(self, line: int) -> int:
        return lib().moe_ring_line_ptr(self.handle, int(line)) or 0

    def wait_ready(self, lines: Sequence[int], stream=None):
        arr = (ctypes.c_int32 * len(lines))(*lines)
        check(lib().moe_ring_wait_ready(self.handle, arr, len(lines), _stream(stream)),
              "moe_ring_wait_ready")

    def release(self, lines: Sequence[int], stream=None):
        arr = (ctypes.c_int32 * len(lines))(*lines)
        check(lib().moe_ring_release(self.handle, arr, len(lines), _stream(stream)),
              "moe_ring_release")

    def close(self):
        if getattr(self, "handle", None) is not None and self.handle.value:
            lib().moe_ring_destroy(self.handle)
            self.handle = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def moe_stage_experts(ring: Ring, layer_id: int, experts: Sequence[int], copy_stream=None):
    """Stage experts into ring lines; returns the line of each expert (held until released)."""
    n = len(experts)
    ex = (ctypes.c_int32 * max(n, 1))(*[int(e) for e in experts])
    out = (ctypes.c_int32 * max(n, 1))()
    check(lib().moe_stage_experts(ring.handle, int(layer_id), ex, n, _stream(copy_stream), out),
          "moe_stage_experts")
    return [out[i] for i in range(n)]


class Layer:
    """One layer as the library sees it (moe_layer) plus the tensors its pointers refer to.

    expert_lines: a device tensor [E, line_elems] of resident lines, or a list with one
    device line (1-D tensor) or None (offloaded, staged through `ring`) per expert.
    """

    def __init__(self, sh: MoeShape, w_router, router_bias, expert_lines, w_gu_shared=None,
                 w_down_shared=None, ring: Optional[Ring] = None, layer_id: int = 0):
        dt = _torch_dtype(sh.dtype)
        E, d = sh.n_experts, sh.d
        _need(w_router, "w_router", dt, (E, d))
        if router_bias is not None:
            _need(router_bias, "router_bias", torch.float32, (E,))
        if isinstance(expert_lines, torch.Tensor):
            _need(expert_lines, "expert_lines", dt, (E, line_elems(sh)))
            rows = [expert_lines[e] for e in range(E)]
        else:
            rows = list(expert_lines)
            if len(rows) != E:
                raise ValueError("expert_lines needs one entry per expert")
            for e, r in enumerate(rows):
                if r is not None:
                    _need(r, f"expert_lines[{e}]", dt, (line_elems(sh),))
        if sh.inter_shared:
            _need(w_gu_shared, "w_gu_shared", dt, (2 * sh.inter_shared, d))
            _need(w_down_shared, "w_down_shared", dt, (d, sh.inter_shared))
        self.shape = sh
        self.ring = ring
        self.layer_id = int(layer_id)
        self._keep = [w_router, router_bias, expert_lines, w_gu_shared, w_down_shared]
        self._ptrs = (ctypes.c_void_p * E)(*[None if r is None else r.data_ptr() for r in rows])
        self.c = MoeLayer(sh, w_router.data_ptr(),
                          router_bias.data_ptr() if router_bias is not None else None,
                          ctypes.cast(self._ptrs, ctypes.POINTER(ctypes.c_void_p)),
                          w_gu_shared.data_ptr() if sh.inter_shared else None,
                          w_down_shared.data_ptr() if sh.inter_shared else None,
                          ring.handle.value if ring is not None else None, self.layer_id)

    @classmethod
    def from_params(cls, params: dict, sh: MoeShape, device="cuda",
                    offloaded: Iterable[int] = (), ring: Optional[Ring] = None,
                    layer_id: int = 0) -> "Layer":
        """Place a layer's parameters (dict of tensors as produced by the input generator):
        resident expert lines in one device tensor, offloaded ones in a pinned host bank
        bound to `ring` under `layer_id`."""
        E = sh.n_experts
        off = sorted(set(int(e) for e in offloaded))
        if off and ring is None:
            raise ValueError("offloaded experts need a ring")
        lines = params["lines"]
        res = [e for e in range(E) if e not in set(off)]
        dev = lambda t: None if t is None else t.to(device).contiguous()
        if not off:
            expert_lines = dev(lines)
        else:
            dl = lines[res].to(device).contiguous() if res else None
            expert_lines = [None] * E
            for i, e in enumerate(res):
                expert_lines[e] = dl[i]
            bank = torch.empty((len(off), lines.shape[1]), dtype=lines.dtype, pin_memory=True)
            bank.copy_(lines[off].to("cpu"))
            slot = [-1] * E
            for i, e in enumerate(off):
                slot[e] = i
            ring.bind_bank(layer_id, bank, slot)
        layer = cls(sh, dev(params["w_router"]), dev(params["router_bias"]), expert_lines,
                    dev(params["w_gu_shared"]), dev(params["w_down_shared"]), ring, layer_id)
        if off:
            layer._keep.append(dl)
        return layer


def moe_prefill_route(layer: Layer, x: torch.Tensor, chunk: int, stream=None) -> dict:
    """Router + top-k + per-chunk histogram. Returns ids, weights, chunk_counts, logits."""
    sh = layer.shape
    T = x.shape[0]
    _need(x, "x", _torch_dtype(sh.dtype), (T, sh.d))
    E, k = sh.n_experts, sh.top_k
    dev = x.device
    n_chunks = (T + chunk - 1) // chunk if chunk > 0 else 0
    r = {
        "ids": torch.empty((T, k), dtype=torch.int32, device=dev),
        "weights": torch.empty((T, k), dtype=torch.float32, device=dev),
        "chunk_counts": torch.empty((n_chunks, E), dtype=torch.int32, device=dev),
        "logits": torch.empty((T, E), dtype=torch.float32, device=dev),
    }
    check(lib().moe_prefill_route(ctypes.byref(layer.c), _vp(x), T, int(chunk), _vp(r["ids"]),
                                  _vp(r["weights"]), _vp(r["chunk_counts"]), _vp(r["logits"]),
                                  _stream(stream)), "moe_prefill_route")
    return r


def moe_prefill_chunk(layer: Layer, x, ids, weights, t0: int, n: int, out, workspace,
                      counts_host=None, stream=None, copy_stream=None) -> None:
    """Expert-major prefill of rows [t0, t0+n) into out (see moe_prefill_chunk in the header)."""
    sh = layer.shape
    T = x.shape[0]
    dt = _torch_dtype(sh.dtype)
    _need(x, "x", dt, (T, sh.d))
    _need(out, "out", dt, (T, sh.d))
    _need(ids, "ids", torch.int32, (T, sh.top_k))
    _need(weights, "weights", torch.float32, (T, sh.top_k))
    ch = None
    if counts_host is not None:
        ch = (ctypes.c_int32 * sh.n_experts)(*[int(v) for v in counts_host])
    check(lib().moe_prefill_chunk(ctypes.byref(layer.c), _vp(x), _vp(ids), _vp(weights), T,
                                  int(t0), int(n), ch, _vp(out), _vp(workspace),
                                  workspace.numel() if workspace is not None else 0,
                                  _stream(stream),
                                  _stream(copy_stream) if copy_stream is not None else None),
          "moe_prefill_chunk")


def moe_noalloc_workspace_bytes() -> int:
    return int(lib().moe_noalloc_workspace_bytes())


def moe_prefill_chunk_noalloc(layer: Layer, x, ids, weights, t0: int, n: int, out,
                              stream=None) -> None:
    """moe_prefill_chunk with the library's own per-device workspace (see the header):
    resident experts only; allocates nothing."""
    sh = layer.shape
    T = x.shape[0]
    dt = _torch_dtype(sh.dtype)
    _need(x, "x", dt, (T, sh.d))
    _need(out, "out", dt, (T, sh.d))
    _need(ids, "ids", torch.int32, (T, sh.top_k))
    _need(weights, "weights", torch.float32, (T, sh.top_k))
    check(lib().moe_prefill_chunk_noalloc(ctypes.byref(layer.c), _vp(x), _vp(ids), _vp(weights),
                                          T, int(t0), int(n), _vp(out), _stream(stream)),
          "moe_prefill_chunk_noalloc")


def layer_buffers(layer: Layer, T: int, chunk: int, device="cuda") -> dict:
    """Output, routing and workspace tensors for moe_prefill_layer over T tokens."""
    sh = layer.shape
    E, k = sh.n_experts, sh.top_k
    n_chunks = (T + chunk - 1) // chunk if chunk > 0 else 0
    return {
        "out": torch.empty((T, sh.d), dtype=_torch_dtype(sh.dtype), device=device),
        "ids": torch.empty((T, k), dtype=torch.int32, device=device),
        "weights": torch.empty((T, k), dtype=torch.float32, device=device),
        "chunk_counts": torch.empty((n_chunks, E), dtype=torch.int32, device=device),
        "logits": torch.empty((T, E), dtype=torch.float32, device=device),
        "workspace": torch.empty(moe_layer_workspace_bytes(sh, max(T, 0), chunk),
                                 dtype=torch.uint8, device=device),
    }


def moe_prefill_layer(layer: Layer, x, chunk: int, workspace=None, out=None, stream=None,
                      copy_stream=None, bufs: Optional[dict] = None) -> dict:
    """Route and run every chunk of the prompt; returns out and the routing tensors.
    bufs: tensors from layer_buffers() to reuse (no allocation per call)."""
    sh = layer.shape
    T = x.shape[0]
    dt = _torch_dtype(sh.dtype)
    _need(x, "x", dt, (T, sh.d))
    if bufs is None:
        bufs = layer_buffers(layer, T, chunk, x.device)
    if workspace is None:
        workspace = bufs["workspace"]
    if out is None:
        out = bufs["out"]
    r = {key: bufs[key] for key in ("ids", "weights", "chunk_counts", "logits")}
    r["out"] = out
    check(lib().moe_prefill_layer(ctypes.byref(layer.c), _vp(x), T, int(chunk), _vp(r["ids"]),
                                  _vp(r["weights"]), _vp(r["chunk_counts"]), _vp(r["logits"]),
                                  _vp(out), _vp(workspace), workspace.numel(), _stream(stream),
                                  _stream(copy_stream) if copy_stream is not None else None),
          "moe_prefill_layer")
    return r


def moe_prefill_stack(layers: Sequence[Layer], x, chunk: int, eps: float, stream=None,
                      copy_stream=None, keep_inputs: bool = False) -> dict:
    """A stack of layers joined by RMSNorm and a residual add, every step in the library:
    h_0 = rmsnorm(x); x_{l+1} = x_l + layer_l(h_l); h_{l+1} = rmsnorm(x_{l+1}).
    Returns {"out": final residual stream}; with keep_inputs also per-layer lists "x" (x_l),
    "inputs" (h_l), "outs" (layer_l(h_l)), "ids", "weights", "logits"."""
    if not layers:
        raise ValueError("empty stack")
    T = x.shape[0]
    xs = x.clone()
    normed = torch.empty_like(x)
    moe_add_rmsnorm(xs, None, eps, normed=normed, stream=stream)
    bufs = layer_buffers(layers[0], T, chunk, x.device)
    keys = ("x", "inputs", "outs", "ids", "weights", "logits")
    res = {key: [] for key in keys}
    for L in layers:
        if keep_inputs:
            res["x"].append(xs.clone())
            res["inputs"].append(normed.clone())
        r = moe_prefill_layer(L, normed, chunk, stream=stream, copy_stream=copy_stream, bufs=bufs)
        if keep_inputs:
            for key, src in (("outs", "out"), ("ids", "ids"), ("weights", "weights"),
                             ("logits", "logits")):
                res[key].append(r[src].clone())
        moe_add_rmsnorm(xs, r["out"], eps, x_out=xs, normed=normed, stream=stream)
    res["out"] = xs
    return res


def moe_set_option(name: str, value: int) -> None:
    """moe_set_option by name: "fused_gu_down" (MOE_OPT_FUSED_GU_DOWN)."""
    from ._abi import OPTIONS
    check(lib().moe_set_option(OPTIONS[name], int(value)), "moe_set_option")


def moe_get_option(name: str) -> int:
    from ._abi import OPTIONS
    v = ctypes.c_int32(0)
    check(lib().moe_get_option(OPTIONS[name], ctypes.byref(v)), "moe_get_option")
    return int(v.value)


def moe_profile_enable(on: bool = True) -> None:
    check(lib().moe_profile_enable(1 if on else 0), "moe_profile_enable")


def moe_profile_read(reset: bool = True, clocks: bool = False) -> dict:
    """{stage: (milliseconds, launches)} of the kernels timed since the last reset; with
    clocks, {stage: (milliseconds, launches, mean shader clock MHz or 0)}."""
    from ._abi import STAGES, MoeProfile
    p = MoeProfile()
    check(lib().moe_profile_read(ctypes.byref(p), 1 if reset else 0), "moe_profile_read")
    if clocks:
        return {name: (p.ms[i], p.launches[i], p.clock_mhz[i]) for i, name in enumerate(STAGES)}
    return {name: (p.ms[i], p.launches[i]) for i, name in enumerate(STAGES)}


def moe_add_rmsnorm(x, delta, eps: float, x_out=None, normed=None, stream=None):
    """x_new = x + delta (if delta given); normed = rmsnorm(x_new). Returns (x_new, normed)."""
    T, d = x.shape
    dt = MOE_BF16 if x.dtype == torch.bfloat16 else MOE_F32
    _need(x, "x", x.dtype, (T, d))
    if delta is not None:
        _need(delta, "delta", x.dtype, (T, d))
        if x_out is None:
            x_out = torch.empty_like(x)
    if normed is None:
        normed = torch.empty_like(x)
    check(lib().moe_add_rmsnorm(_vp(x), _vp(delta), T, d, dt, float(eps), _vp(x_out),
                                _vp(normed), _stream(stream)), "moe_add_rmsnorm")
    return (x_out if delta is not None else x), normed
