"""C-ABI checks that need no GPU: the library loads, exports every function the header
declares, the ctypes table matches the header, and argument validation rejects bad calls
before anything touches the device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_prefill.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s*(moe_[a-z_0-9]+)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def abi():
    from routed_expert_grouped_moe_amd import _abi
    if not os.path.exists(_abi.LIB_PATH):
        import routed_expert_grouped_moe_amd.build as b
        b.build()
    return _abi


def test_header_parses():
    names = _declared_functions()
    assert "moe_prefill_route" in names and "moe_prefill_chunk" in names
    assert "moe_stage_experts" in names
    assert len(names) >= 18


def test_every_declared_symbol_is_exported(abi):
    raw = ctypes.CDLL(abi.LIB_PATH)
    missing = [n for n in _declared_functions() if not hasattr(raw, n)]
    assert not missing, missing


def test_ctypes_table_matches_header(abi):
    assert sorted(abi.SIGNATURES) == _declared_functions()
    abi.lib()   # applies every signature


def test_version_and_status_strings(abi):
    L = abi.lib()
    assert L.moe_abi_version() == 7
    assert L.moe_status_string(abi.MOE_OK) == b"MOE_OK"
    assert L.moe_status_string(abi.MOE_ERR_WORKSPACE) == b"MOE_ERR_WORKSPACE"
    assert L.moe_status_string(99) == b"MOE_ERR_UNKNOWN"


def test_options(abi):
    L = abi.lib()
    v = ctypes.c_int32(-1)
    assert L.moe_get_option(abi.OPTIONS["fused_gu_down"], ctypes.byref(v)) == abi.MOE_OK
    assert v.value == 0                     # off until set
    assert L.moe_set_option(abi.OPTIONS["fused_gu_down"], 7) == abi.MOE_OK
    assert L.moe_get_option(abi.OPTIONS["fused_gu_down"], ctypes.byref(v)) == abi.MOE_OK
    assert v.value == 1
    assert L.moe_set_option(abi.OPTIONS["fused_gu_down"], 0) == abi.MOE_OK
    assert L.moe_set_option(99, 1) == abi.MOE_ERR_INVALID
    assert b"option" in L.moe_last_error()
    assert L.moe_get_option(abi.OPTIONS["fused_gu_down"], None) == abi.MOE_ERR_INVALID


def _shape(abi, d=128, E=8, k=2, I=64, Is=64, dt=0):
    return abi.MoeShape(d, E, k, I, Is, dt)


def test_workspace_bytes(abi):
    L = abi.lib()
    sh = _shape(abi)
    w1 = L.moe_workspace_bytes(ctypes.byref(sh), 1)
    w100 = L.moe_workspace_bytes(ctypes.byref(sh), 100)
    assert 0 < w1 < w100
    # fp32 intermediates are wider than bf16
    assert L.moe_workspace_bytes(ctypes.byref(_shape(abi, dt=1)), 100) > w100
    for bad in (_shape(abi, d=96), _shape(abi, d=32), _shape(abi, E=0), _shape(abi, k=9),
                _shape(abi, I=100), _shape(abi, Is=32), _shape(abi, dt=7), _shape(abi, E=1025)):
        assert L.moe_workspace_bytes(ctypes.byref(bad), 10) == 0
    assert L.moe_workspace_bytes(ctypes.byref(sh), -1) == 0
    o = abi.MoeWsOffsets()
    assert L.moe_workspace_offsets(ctypes.byref(sh), 100, ctypes.byref(o)) == abi.MOE_OK
    assert o.total == w100
    assert o.counts < o.offsets < o.row_tok < o.row_slot < o.total
    assert all(v % 256 == 0 for v in (o.counts, o.offsets, o.row_tok, o.row_slot))


def test_layer_workspace_bytes(abi):
    """A layer call's workspace for up-front bucketing and the deferred shared down + combine:
    the one-chunk workspace, one block of member lists per chunk (the one-chunk layout's
    block histograms through row_slot: from after the expert-line table up to h) and a second
    h_shared block for a chunk's rows; no extra block without a shared expert, nothing extra
    for a single chunk."""
    L = abi.lib()

    def size(sh, T, chunk):
        return L.moe_layer_workspace_bytes(ctypes.byref(sh), T, chunk)

    for Is in (64, 0):
        sh = _shape(abi, Is=Is)
        E = sh.n_experts
        base = L.moe_workspace_bytes(ctypes.byref(sh), 100)
        o = abi.MoeWsOffsets()
        assert L.moe_workspace_offsets(ctypes.byref(sh), 100, ctypes.byref(o)) == abi.MOE_OK
        stride = o.h - -(-8 * E // 256) * 256          # lists: after the line table, up to h
        second = o.y - o.h_shared
        assert second == (-(-100 * Is * 2 // 256) * 256 if Is else 0)    # bf16 rows of I_s
        assert size(sh, 100, 100) == base
        assert size(sh, 60, 100) == L.moe_workspace_bytes(ctypes.byref(sh), 60)
        assert size(sh, 0, 100) == L.moe_workspace_bytes(ctypes.byref(sh), 1)
        for T in (101, 200, 201, 1000):
            n_chunks = -(-T // 100)
            assert size(sh, T, 100) == base + n_chunks * stride + second, (Is, T)
    sh = _shape(abi)
    assert size(sh, 100, 0) == 0 and size(sh, -1, 10) == 0
    assert size(_shape(abi, d=96), 200, 100) == 0


def test_validation_before_device_work(abi):
    """Bad arguments return MOE_ERR_INVALID with a message and enqueue nothing (no GPU here,
    so any device call would fail differently)."""
    L = abi.lib()
    assert L.moe_prefill_route(None, None, 0, 1, None, None, None, None, None) == abi.MOE_ERR_INVALID
    assert b"layer" in L.moe_last_error()
    sh = _shape(abi, d=100)
    layer = abi.MoeLayer(sh, 16, None, None, None, None, None, 0)
    assert L.moe_prefill_route(ctypes.byref(layer), None, 4, 1, None, None, None, None, None) == abi.MOE_ERR_INVALID
    assert b"d=100" in L.moe_last_error()
    sh = _shape(abi)
    layer = abi.MoeLayer(sh, 256, None, None, 512, 1024, None, 0)
    # chunk < 1
    assert L.moe_prefill_route(ctypes.byref(layer), 4096, 4, 0, 64, 64, 64, 64, None) == abi.MOE_ERR_INVALID
    # T == 0 is a valid no-op
    assert L.moe_prefill_route(ctypes.byref(layer), None, 0, 1, None, None, None, None, None) == abi.MOE_OK
    # misaligned x
    assert L.moe_prefill_route(ctypes.byref(layer), 4097, 4, 1, 64, 64, 64, 64, None) == abi.MOE_ERR_INVALID
    # chunk: NULL expert table
    assert L.moe_prefill_chunk(ctypes.byref(layer), 4096, 64, 64, 4, 0, 4, None, 4096, 4096, 1 << 20, None, None) == abi.MOE_ERR_INVALID
    # chunk: rows out of range
    lines = (ctypes.c_void_p * 8)(*([1 << 20] * 8))
    layer.expert_lines = ctypes.cast(lines, ctypes.POINTER(ctypes.c_void_p))
    assert L.moe_prefill_chunk(ctypes.byref(layer), 4096, 64, 64, 4, 2, 3, None, 4096, 4096, 1 << 20, None, None) == abi.MOE_ERR_INVALID
    # chunk: an expert with no line and no ring
    lines[3] = None
    assert L.moe_prefill_chunk(ctypes.byref(layer), 4096, 64, 64, 4, 0, 4, None, 4096, 4096, 1 << 20, None, None) == abi.MOE_ERR_RING
    lines[3] = 1 << 20
    # chunk: workspace too small (checked before any launch)
    assert L.moe_prefill_chunk(ctypes.byref(layer), 4096, 64, 64, 4, 0, 4, None, 4096, 4096, 100, None, None) == abi.MOE_ERR_WORKSPACE
    assert b"workspace" in L.moe_last_error()
    # n == 0 is a valid no-op
    assert L.moe_prefill_chunk(ctypes.byref(layer), 4096, 64, 64, 4, 4, 0, None, 4096, 4096, 0, None, None) == abi.MOE_OK
    # shared expert declared but missing weights
    layer2 = abi.MoeLayer(sh, 256, None, ctypes.cast(lines, ctypes.POINTER(ctypes.c_void_p)), None, None, None, 0)
    assert L.moe_prefill_chunk(ctypes.byref(layer2), 4096, 64, 64, 4, 0, 4, None, 4096, 4096, 1 << 30, None, None) == abi.MOE_ERR_INVALID


def test_ring_and_rmsnorm_validation(abi):
    L = abi.lib()
    out = ctypes.c_void_p(1)
    sh = _shape(abi)
    assert L.moe_ring_create(ctypes.byref(sh), None, 4, ctypes.byref(out)) == abi.MOE_ERR_INVALID
    assert out.value is None
    assert L.moe_ring_create(ctypes.byref(sh), 4096 + 16, 4, ctypes.byref(out)) == abi.MOE_ERR_INVALID
    assert L.moe_ring_create(ctypes.byref(sh), 4096, 0, ctypes.byref(out)) == abi.MOE_ERR_INVALID
    bad = _shape(abi, k=0)
    assert L.moe_ring_create(ctypes.byref(bad), 4096, 4, ctypes.byref(out)) == abi.MOE_ERR_INVALID
    L.moe_ring_destroy(None)   # NULL-safe
    assert L.moe_ring_line_ptr(None, 0) is None
    assert L.moe_stage_experts(None, 0, None, 0, None, None) == abi.MOE_ERR_INVALID
    assert L.moe_add_rmsnorm(None, None, 4, 64, 0, 1e-6, None, None, None) == abi.MOE_ERR_INVALID
    assert L.moe_add_rmsnorm(4096, None, 4, 64, 0, -1.0, None, 4096, None) == abi.MOE_ERR_INVALID
    assert L.moe_add_rmsnorm(4096, None, 0, 64, 0, 1e-6, None, 4096, None) == abi.MOE_OK


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    """The product path has no fallback: with the library missing, calls raise."""
    from routed_expert_grouped_moe_amd import _abi
    monkeypatch.setattr(_abi, "_lib", None)
    monkeypatch.setattr(_abi, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(RuntimeError, match="build the HIP library"):
        _abi.lib()
