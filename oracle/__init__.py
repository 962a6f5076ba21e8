"""TEST INFRASTRUCTURE: the CPU oracle of the routed-attention layer.

Only the tests, the package smoke check and the benchmark's CPU-baseline leg
may import this package.  The product path never does.
"""
