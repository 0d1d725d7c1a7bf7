"""fp64 CPU oracle for GQA decode attention.

TEST INFRASTRUCTURE: only the tests, the smoke check and the benchmark's
CPU-baseline leg import this package.  The product path (the HIP library and
its Python binding) never imports or calls it.
"""
from . import bruteforce, reference  # noqa: F401
from .reference import *  # noqa: F401,F403
