"""Test infrastructure: the fp64 CPU oracle for the group-circulant (EQ-Linear) layer.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg use this
package. The product path (the HIP library and its binding) never imports it.
The p4m (dihedral D4) layer's oracle is the submodule `oracle.p4m_oracle`.
"""
from .eqlinear_oracle import (  # noqa: F401
    unroll,
    fwd,
    bwd_x,
    bwd_w,
    half_spectrum,
    gelu,
    fwd_fused,
    gelu_grad,
    fused_epilogue_bwd,
    real_gemm_count,
    actual_flops,
    dense_equivalent_flops,
)
