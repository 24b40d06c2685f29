"""MI355X-native DSA (DeepSeek Sparse Attention) decode path.

``sparse_attention_05_amd.dsa`` is the Python binding of the C-ABI library
``libdsa.so`` (hand-written HIP for gfx950); ``inputs`` makes seeded
synthetic workloads. Importing the package itself loads nothing.
"""
__all__ = ["dsa", "inputs"]
