"""MI355X-native HySparse2 inner-level attention (token-level sparse KV reuse).

The compute path lives in the HIP library ``libhs2.so`` behind the C ABI of
``include/hs2.h``; ``token_level_sparse_full_amd.hs2`` is its thin ctypes
binding.  Importing this package does not load the library.
"""
