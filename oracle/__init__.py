"""fp64 CPU oracle for the LatentMoE layer forward -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the package-level smoke check and the benchmark's
CPU-baseline leg may import or call anything in this package.  The product
path (the HIP library and its Python binding) never does, and shares no code
with it: this package imports nothing from the product package, and decodes
every stored byte (bf16, E4M3, E2M1) with its own code.

Method: "Nemotron 3 Super: Open, Efficient Mixture-of-Experts Hybrid
Mamba-Transformer Model for Agentic Reasoning", section 3.2 (LatentMoE) and the
section 3.1 shape table; FP4 storage per the same page's section 3.6 (dual
scale) and "Nemotron 3 Ultra" (E2M1 values, E4M3 block scales); the shared
expert in the same FP4 format and W_down / W_up as per-tensor FP8 per the
released precision mix ("Nemotron 3.5 Super and Lightning", 4-bit
quantisation section).

`ssm` holds the Mamba-2 state recurrence used to check the checkpoint + replay
verification kernels ("Nemotron 3.5 Super and Lightning", serving section).

Every function here is pinned by the CPU tests (closed forms, special cases
that reduce to a textbook mixture, brute force on tiny inputs, exhaustive
format tables).  Nothing here is pinned against values printed on the pages:
the pages print no numeric LatentMoE example.
"""
from .formats import bf16_to_f64, e2m1_to_f64, e4m3fn_to_f64, fp4_dequant, fp8_dequant  # noqa: F401
from . import ssm  # noqa: F401
from .latentmoe import (  # noqa: F401
    expert_ffn,
    forward,
    projection_weights,
    router_logits,
    select_topk,
    shared_expert,
    shared_weights,
    softmax_selected,
    topk_gap,
)
