"""Oracle package -- TEST INFRASTRUCTURE ONLY (see r2l_oracle.py).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The library and its binding never do.
"""
from .r2l_oracle import *  # noqa: F401,F403
