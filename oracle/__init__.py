"""CPU oracle for the one-GPU Mega MoE forward.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
baseline may import or call anything in this package; the product path (the HIP
library and its binding) never does, and this package never imports the product.
"""
from .moe_oracle import *  # noqa: F401,F403
from .gemm_oracle import *  # noqa: F401,F403
