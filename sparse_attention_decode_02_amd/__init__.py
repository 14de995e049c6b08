"""MI355X-native paged DSA step: indexer scores, length-bounded exact top-k,
GQA sparse attention split over the k slots, and the log-sum-exp merge, as
hand-written HIP kernels for gfx950 behind a C-ABI library (libdsa.so).

Importing the package loads nothing; ``sparse_attention_decode_02_amd.lib``
loads the built library and raises if it is missing.
"""

__all__ = ["inputs", "lib", "build"]
