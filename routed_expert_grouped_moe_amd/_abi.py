"""ctypes view of include/moe_prefill.h: structs, status codes and function signatures.

Loading fails loudly when the HIP library has not been built: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoeprefill.so")

MOE_OK, MOE_ERR_INVALID, MOE_ERR_WORKSPACE, MOE_ERR_RING, MOE_ERR_HIP, MOE_ERR_UNSUPPORTED = range(6)
MOE_BF16, MOE_F32 = 0, 1

c_i32, c_i64, c_f32, c_vp, c_sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t


class MoeShape(ctypes.Structure):
    _fields_ = [("d", c_i32), ("n_experts", c_i32), ("top_k", c_i32), ("inter", c_i32),
                ("inter_shared", c_i32), ("dtype", c_i32)]


class MoeLayer(ctypes.Structure):
    _fields_ = [("shape", MoeShape), ("w_router", c_vp), ("router_bias", c_vp),
                ("expert_lines", ctypes.POINTER(c_vp)), ("w_gu_shared", c_vp),
                ("w_down_shared", c_vp), ("ring", c_vp), ("layer_id", c_i32)]


class MoeWsOffsets(ctypes.Structure):
    _fields_ = [("counts", c_sz), ("offsets", c_sz), ("row_tok", c_sz), ("row_slot", c_sz),
                ("h", c_sz), ("h_shared", c_sz), ("y", c_sz), ("total", c_sz)]


class MoeProfile(ctypes.Structure):
    _fields_ = [("version", c_i32), ("n_stages", c_i32), ("ms", ctypes.c_double * 32),
                ("launches", c_i64 * 32), ("clock_mhz", ctypes.c_double * 32)]


STAGES = ["router", "topk", "chunk_counts", "table", "hist", "scan", "permute", "gu_shared",
          "down_shared", "gu_routed", "down_routed", "combine", "rmsnorm", "down_shared_combine",
          "gu_mixed", "gu_down_fused", "down_mixed"]

OPTIONS = {"fused_gu_down": 1}       # MOE_OPT_* of include/moe_prefill.h


COPY_KINDS = ["initial", "ahead", "demand", "cross_layer"]     # MOE_COPY_* order


class MoeRingStats(ctypes.Structure):
    _fields_ = [("version", c_i32), ("n_lines", c_i32), ("hits", c_i64), ("misses", c_i64),
                ("bytes_h2d", c_i64), ("copy_waits", c_i64), ("waves", c_i64),
                ("requested_bytes", c_i64 * 4), ("copied_bytes", c_i64 * 4),
                ("pinned_uses", c_i64)]


# name -> (restype, argtypes); every function declared in include/moe_prefill.h
SIGNATURES = {
    "moe_abi_version": (c_i32, []),
    "moe_status_string": (ctypes.c_char_p, [c_i32]),
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_workspace_bytes": (c_sz, [ctypes.POINTER(MoeShape), c_i64]),
    "moe_layer_workspace_bytes": (c_sz, [ctypes.POINTER(MoeShape), c_i64, c_i64]),
    "moe_workspace_offsets": (c_i32, [ctypes.POINTER(MoeShape), c_i64,
                                      ctypes.POINTER(MoeWsOffsets)]),
    "moe_prefill_route": (c_i32, [ctypes.POINTER(MoeLayer), c_vp, c_i64, c_i64, c_vp, c_vp,
                                  c_vp, c_vp, c_vp]),
    "moe_prefill_chunk": (c_i32, [ctypes.POINTER(MoeLayer), c_vp, c_vp, c_vp, c_i64, c_i64,
                                  c_i64, c_vp, c_vp, c_vp, c_sz, c_vp, c_vp]),
    "moe_noalloc_workspace_bytes": (c_sz, []),
    "moe_prefill_chunk_noalloc": (c_i32, [ctypes.POINTER(MoeLayer), c_vp, c_vp, c_vp, c_i64,
                                          c_i64, c_i64, c_vp, c_vp]),
    "moe_prefill_layer": (c_i32, [ctypes.POINTER(MoeLayer), c_vp, c_i64, c_i64, c_vp, c_vp,
                                  c_vp, c_vp, c_vp, c_vp, c_sz, c_vp, c_vp]),
    "moe_ring_create": (c_i32, [ctypes.POINTER(MoeShape), c_vp, c_i32, ctypes.POINTER(c_vp)]),
    "moe_ring_bind_bank": (c_i32, [c_vp, c_i32, c_vp, c_vp]),
    "moe_stage_experts": (c_i32, [c_vp, c_i32, c_vp, c_i32, c_vp, c_vp]),
    "moe_ring_prefetch": (c_i32, [c_vp, c_i32, c_vp, c_i32, c_vp]),
    "moe_ring_wait_ready": (c_i32, [c_vp, c_vp, c_i32, c_vp]),
    "moe_ring_release": (c_i32, [c_vp, c_vp, c_i32, c_vp]),
    "moe_ring_line_ptr": (c_vp, [c_vp, c_i32]),
    "moe_ring_stats": (c_i32, [c_vp, ctypes.POINTER(MoeRingStats)]),
    "moe_ring_reset_stats": (c_i32, [c_vp]),
    "moe_ring_invalidate": (c_i32, [c_vp]),
    "moe_ring_destroy": (None, [c_vp]),
    "moe_profile_enable": (c_i32, [c_i32]),
    "moe_set_option": (c_i32, [c_i32, c_i32]),
    "moe_get_option": (c_i32, [c_i32, ctypes.POINTER(c_i32)]),
    "moe_profile_read": (c_i32, [ctypes.POINTER(MoeProfile), c_i32]),
    "moe_add_rmsnorm": (c_i32, [c_vp, c_vp, c_i64, c_i32, c_i32, c_f32, c_vp, c_vp, c_vp]),
}

_lib = None


ABI_VERSION = 7     # MOE_ABI_VERSION of include/moe_prefill.h


def lib():
    """The loaded libmoeprefill.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build the HIP library first "
                "(python -m routed_expert_grouped_moe_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        if L.moe_abi_version() != ABI_VERSION:
            raise RuntimeError(f"{LIB_PATH} has ABI version {L.moe_abi_version()}, the binding "
                               f"expects {ABI_VERSION}: rebuild the HIP library")
        _lib = L
    return _lib


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        L = lib()
        self.status = status
        msg = L.moe_last_error().decode(errors="replace")
        name = L.moe_status_string(status).decode()
        super().__init__(f"{where}: {name}: {msg}")


def check(status: int, where: str) -> None:
    if status != MOE_OK:
        raise MoeError(status, where)
