"""CPU oracle of the LSA decode hot path: test infrastructure only.

Only the tests, the smoke check and the benchmark's CPU-baseline leg import
this package.  The product library never links or calls it.
"""
