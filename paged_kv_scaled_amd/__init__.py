"""paged_kv_scaled_amd: scaled dot-product attention over a paged KV cache on MI355X.

The computation lives in libpkv.so (hand-written HIP for gfx950, C ABI in
include/pkv.h); `binding` marshals torch tensors into it and `workloads` draws
seeded synthetic inputs.  Importing the package loads nothing.
"""
__all__ = ["binding", "workloads", "build"]
