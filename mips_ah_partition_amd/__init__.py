"""MI355X-native asymmetric-hashing (AH) maximum-inner-product search path.

Submodules
  ahlib   -- thin ctypes binding of the C ABI (include/ah.h, libah.so)
  index   -- host-side index build: partition k-means, anisotropic codebooks,
             coupled encoding, leaf sort
  search  -- AHIndex: search_batched over the four C-ABI calls
  costs   -- per-query operation and byte counts of the path
Submodules are imported on demand so that host-only tools do not load the GPU
library.
"""
__all__ = ["ahlib", "index", "search", "costs"]
