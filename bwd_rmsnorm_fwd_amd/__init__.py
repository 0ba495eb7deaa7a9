"""Fused row-wise RMSNorm for AMD MI355X (gfx950): forward, explicit backward,
residual-add + RMSNorm, and a split-row decode path, as hand-written HIP
kernels behind a C ABI (include/rmsnorm.h).

Importing the package loads nothing; ``bwd_rmsnorm_fwd_amd.binding`` loads
the compiled library on first use and raises if it is missing.
"""
