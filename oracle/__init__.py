"""fp64 CPU oracle of the bidirectional SSD scan (and of the hybrids'
attention layer, attention.py) -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the bench's CPU-baseline leg may import
this package.  The GPU library never links, loads or calls it.
"""
