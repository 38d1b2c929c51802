"""MI355X-native RocketKV hot path: SnapKV eviction + Hybrid Sparse Attention decode.

The compute path is the C-ABI library ``librocketkv.so`` (hand-written HIP for
gfx950) declared in ``include/rocketkv.h``.  ``sparse_decode_attention_amd.rocketkv``
is its thin ctypes binding; importing it loads the library and fails loudly if
it has not been built.  Importing this package itself loads nothing.
"""

__all__ = ["rocketkv", "workloads"]
