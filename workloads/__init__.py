"""Seeded synthetic inputs for one expert-parallel rank's MoE expert step.

This package only draws random numbers and stores them in the storage formats the
step consumes (fp32, bfloat16 bits, OCP fp8 e4m3 codes + per-row fp32 scales).  It
holds none of the step's arithmetic: no gather, no FFN, no combine.  Both the HIP
path (through its Python binding) and the CPU oracle read the same arrays from here.
"""
from .gen import (  # noqa: F401
    BASE_SEED,
    C1,
    C2,
    C4,
    C4Setup,
    c2_pool,
    Arrivals,
    Batch,
    LayerWeights,
    ZIPF_P,
    c0_tiny,
    c1_decode,
    c2_skewed_batch,
    c2_weights,
    c4_prefill_setup,
    c4_wave,
    make_layer_weights,
    merge_batches, subset_batch,
    to_bf16_bits,
    to_e4m3_codes,
    zipf_probs,
)
