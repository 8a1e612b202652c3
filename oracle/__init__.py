"""fp64 CPU oracle for the weight-only 4-bit linear layer.

TEST INFRASTRUCTURE: only the tests, the package smoke check and the
benchmark's CPU-baseline leg import this package.  The GPU product path never
imports, links or executes anything in it.

Parity status of each function (what pins it) is listed in the header of
``q4_oracle.c`` and checked by ``tests/test_oracle.py``; no function here is
parity-unpinned.
"""
