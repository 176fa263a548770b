"""sawkv: MI355X (gfx950) fused block-diagonal Hadamard + token-wise INT4
paged KV-cache append, and its dequantise/inverse-rotate read-back.

The compute lives in the HIP library ``libsawkv.so`` (C ABI, declared in
include/sawkv.h). ``int4_kv_cache_amd.sawkv`` is the thin ctypes binding over
it; importing that module loads the library and raises if it is missing.
``int4_kv_cache_amd.workloads`` holds the seeded synthetic inputs and needs no
library.
"""

__all__ = ["sawkv", "workloads"]
