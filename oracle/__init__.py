"""fp64 CPU oracle of the routed-expert MoE deep-prefill layer.

Test infrastructure: only the test-suite, the smoke check and the benchmark's CPU-baseline
leg may import it. The HIP path never does.
"""
from .moe_oracle import *  # noqa: F401,F403
