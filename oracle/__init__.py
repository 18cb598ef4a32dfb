"""CPU oracle for the fused MaxSim path -- TEST INFRASTRUCTURE ONLY.

A plain, slow reference written from the paper "Flash-MaxSim: IO-Aware Fused
Kernels for Late-Interaction Scoring" (arXiv 2605.29517).  Only the tests, the
smoke check and the CPU-baseline leg of the benchmark may import it; the
product path (the HIP library and its binding) never does, and the two share
no code.
"""
from .oracle import (  # noqa: F401
    F16,
    BF16,
    build,
    lib_path,
    f16_to_f64,
    bf16_to_f64,
    fwd_padded,
    fwd_varlen,
    fwd_i8,
    sim_at,
    csr_build,
    bwd,
    num_threads,
    fwd_pairs,
    topk,
    two_stage_topk,
    csr_build_varlen,
    bwd_varlen,
    chamfer_nn,
    chamfer,
    chamfer_loss,
    chamfer_csr,
    chamfer_bwd,
)
