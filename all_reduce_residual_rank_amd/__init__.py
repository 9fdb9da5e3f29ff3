"""MI355X (gfx950) fused rank-sum + residual-add + RMSNorm (+ per-token FP8) epilogue.

The work runs in ``libarrms.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/arrms.h``). ``all_reduce_residual_rank_amd.arrms`` is
the thin ctypes binding; importing it loads the library and fails loudly
when it has not been built. ``all_reduce_residual_rank_amd.workloads``
holds the seeded synthetic inputs and needs no GPU.
"""
__all__ = ["arrms", "workloads"]
