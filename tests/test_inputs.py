"""Seeded input generator: determinism, value recipe, and the Zipf bias calibration."""
import numpy as np
import torch

import moe_inputs as mi
import oracle.moe_oracle as orc


def test_deterministic_and_distinct():
    wl = mi.custom_workload(T=33, d=64, E=8, k=2, inter=64, inter_shared=64)
    a = mi.make_layer(wl, 0)
    b = mi.make_layer(wl, 0)
    c = mi.make_layer(wl, 1)
    for key in ("w_router", "lines", "w_gu_shared", "w_down_shared"):
        assert torch.equal(a[key], b[key])
        assert not torch.equal(a[key], c[key])
    assert torch.equal(mi.make_x(wl), mi.make_x(wl))


def test_shapes_and_scales():
    wl = mi.custom_workload(T=64, d=256, E=16, k=4, inter=128, inter_shared=192)
    p = mi.make_layer(wl)
    sh = wl.shape
    assert p["lines"].shape == (16, 3 * 128 * 256) and p["lines"].dtype == torch.bfloat16
    gu, dn = mi.split_lines(p["lines"], sh)
    assert gu.shape == (16, 256, 256) and dn.shape == (16, 256, 128)
    assert abs(gu.float().std().item() - 1 / np.sqrt(256)) < 0.01
    assert abs(dn.float().std().item() - 1 / np.sqrt(128)) < 0.01
    assert abs(p["w_router"].float().std().item() - 0.02) < 0.002
    assert p["w_gu_shared"].shape == (384, 256) and p["w_down_shared"].shape == (256, 192)
    x = mi.make_x(wl)
    assert x.shape == (64, 256) and abs(x.float().std().item() - 1.0) < 0.05


def test_bf16_bits_roundtrip():
    t = torch.tensor([1.0, -2.0, 3.140625], dtype=torch.bfloat16)
    bits = mi.to_numpy_exact(t)
    assert bits.dtype == np.uint16
    assert np.array_equal(orc.as_f64(bits), [1.0, -2.0, 3.140625])


def test_zipf_calibration_hottest_share():
    """At s = 1.5 (d = 2048, E = 512, k = 8) the hottest expert takes about 10% of slots."""
    wl = mi.WORKLOADS["stack_32700"]
    E, d, k = 512, 2048, 8
    g = torch.Generator().manual_seed(5)
    x = torch.randn(2048, d, generator=g).to(torch.bfloat16)
    w_r = (torch.randn(E, d, generator=g) * mi.ROUTER_STD).to(torch.bfloat16)
    b = mi.zipf_bias(E, 1.5, wl.seed, 0)
    logits = orc.router_logits(mi.to_numpy_exact(x), mi.to_numpy_exact(w_r), b)
    ids = orc.select_topk(logits, k)
    share = np.bincount(ids.ravel(), minlength=E).max() / ids.size
    assert 0.08 <= share <= 0.12, share
    # s = 1.1 with the same lambda is milder
    ids11 = orc.select_topk(orc.router_logits(mi.to_numpy_exact(x), mi.to_numpy_exact(w_r),
                                              mi.zipf_bias(E, 1.1, wl.seed, 0)), k)
    assert np.bincount(ids11.ravel(), minlength=E).max() / ids11.size < share
