"""CPU oracle of the decode-time KV eviction pass (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg import
this package.  The product library never does.
"""
from .oracle import *  # noqa: F401,F403
from .oracle import build, lib  # noqa: F401
