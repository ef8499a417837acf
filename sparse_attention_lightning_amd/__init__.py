"""MI355X-native packed lightning-indexer step (gfx950, HIP).

The work sits behind a C-ABI shared library (``include/idx.h``); the Python
binding in :mod:`sparse_attention_lightning_amd.idx` only marshals arguments
and raises when the library is missing or refuses a call.  The seeded
synthetic inputs live in :mod:`sparse_attention_lightning_amd.workloads`.
"""
