"""Plain CPU oracle of the packed lightning-indexer step.

Test infrastructure only: the tests, the smoke check and the benchmark's
CPU-baseline leg may import it; the library under
``sparse_attention_lightning_amd`` never does.
"""
