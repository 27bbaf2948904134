"""MI355X-native FP4 (NVFP4) KV-cache chunk attention.

The compute path lives in the HIP library libfp4kv.so (C ABI in
include/fp4kv.h); `api` is a thin ctypes binding over it and `workloads`
holds the seeded synthetic workloads.  Importing the package does not load
the library; the first call through `api` does, and fails loudly if it is
not built.
"""
__all__ = ["api", "workloads"]
