"""A8W4 fused mixture-of-experts layer for MI355X (gfx950).

FP8 E4M3 activations with per-1x32 E8M0 scales times MXFP4 weights, BF16
output, computed by hand-written HIP kernels behind the C ABI declared in
``include/moe_a8w4.h``.  ``abi`` binds that library; ``workloads`` draws the
seeded synthetic inputs.  Importing the package loads nothing native.
"""
__all__ = ["abi", "workloads"]
