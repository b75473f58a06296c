"""Fixed-budget ragged pass over a blocked KV cache (Dynamic SplitFuse), MI355X-native.

The product is the C-ABI library ``libfg.so`` (include/fg.h): host composition and block
allocation, a HIP kv_append kernel and a HIP ragged blocked attention kernel for gfx950.
``fg`` is its ctypes binding; ``runtime`` holds the PyTorch-side device plumbing;
``workloads`` generates seeded synthetic passes.
"""
__all__ = ["fg", "runtime", "workloads"]
