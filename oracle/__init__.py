"""CPU oracle of the verify step -- test infrastructure only.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The library under rejection_sampling_amd/ never does.
"""
