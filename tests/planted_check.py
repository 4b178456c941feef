"""Child process of tests/test_gpu_controls.py: loads one planted test build of the library
in place of the real one and runs the parity check aimed at its mistake, on the GPU.

    python -m tests.planted_check <name> <library path>

Prints CONTROL_RED (the check failed, as it must) or CONTROL_GREEN (it passed) and exits 0;
any other exit code is an error of the run itself.
"""
import sys
import traceback


def main(name: str, lib: str) -> int:
    import numpy as np
    import torch

    from routed_expert_grouped_moe_amd import _abi
    _abi.LIB_PATH = lib                       # before the first call loads a library
    import moe_inputs as mi
    import routed_expert_grouped_moe_amd as moe
    from tests import test_gpu_stages as st
    from tests.parity import oracle_params, place

    print(f"[control] {name}: {lib}", flush=True)
    torch.cuda.set_device(0)
    wl = mi.custom_workload("control", T=2000, d=256, E=32, k=4, inter=128, inter_shared=128,
                            zipf_s=1.1, seed=41)
    params = mi.make_layer(wl, device="cuda")
    x = mi.make_x(wl, device="cuda")
    stats = st._new_stats()
    try:
        if name == "combine_desc":          # (iv): zero shared down projection, canonical order
            p0 = dict(params)
            p0["w_down_shared"] = torch.zeros_like(params["w_down_shared"])
            c = st.Chunk(moe, wl, p0, x, 0, 600)
            st._check_out(c, oracle_params(p0, wl), np.arange(600), stats, exact_shared=True)
        elif name == "h_trunc":             # (i): h rounded to nearest even
            c = st.Chunk(moe, wl, params, x, 0, 600)
            st._check_routed(c, oracle_params(params, wl), range(32), stats)
        elif name == "out_twice":           # (iii): one rounding of the whole sum
            c = st.Chunk(moe, wl, params, x, 0, 600)
            st._check_out(c, oracle_params(params, wl), np.arange(600), stats)
        elif name == "korder_tall":         # chunk invariance: 320-row tiles against 64-row ones
            _, L = place(wl, params=params)
            a = moe.moe_prefill_layer(L, x, wl.T)["out"].clone()      # 250 rows per expert
            b = moe.moe_prefill_layer(L, x, 300)["out"]
            torch.cuda.synchronize()
            diff = int((a.view(torch.int16) != b.view(torch.int16)).sum())
            assert diff == 0, f"batched and chunk-300 outputs differ at {diff} elements"
        else:
            print(f"unknown control {name}", flush=True)
            return 2
    except AssertionError as e:
        print(f"CONTROL_RED {name}: {e}", flush=True)
        return 0
    except Exception:
        traceback.print_exc()
        return 3
    print(f"CONTROL_GREEN {name}", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1], sys.argv[2]))
