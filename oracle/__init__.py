"""Independent fp64 CPU oracle for the FNO spectral convolution.

TEST INFRASTRUCTURE ONLY: used by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py.  The HIP library never imports or links it, and
it imports nothing from the library.  Every function is pinned by tests in
tests/test_oracle.py against closed forms, invariants, brute force and a
library FFT; no function here is parity-unpinned.
"""
from .spectral import *  # noqa: F401,F403
from .spectral import __all__  # noqa: F401
