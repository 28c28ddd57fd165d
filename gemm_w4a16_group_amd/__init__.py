"""W4A16 group-quantized linear layer for MI355X (gfx950).

C[M, N] = Wdeq[M, K] . X[K, N] with Wdeq = (q - z) * s, int4 codes q and z,
fp16 scales s, one (s, z) per 128 consecutive k of a row.  The compute path
is the C-ABI library ``libw4a16.so`` (hand-written HIP kernels); the Python
names below only marshal torch device tensors into its entry points.
"""

__all__ = ["pack", "gemv", "gemm", "workspace_size", "plan_default", "Plan", "Workspace", "lib"]


def __getattr__(name):
    # The binding is loaded on first use, so ``gemm_w4a16_group_amd.inputs``
    # can be imported without the shared library.
    if name in __all__ or name in ("W4A16Error", "load_library"):
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
