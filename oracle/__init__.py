"""fp64 CPU oracle for paged decode attention.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the
benchmark's CPU-baseline leg use it.  The product path never imports it,
and it imports nothing from the product package.

The arithmetic lives in ``oracle.c`` (plain C, fp64, OpenMP over
(sequence, KV head) units); ``oracle.py`` builds it with gcc and marshals
numpy arrays across ctypes.
"""
from .oracle import DTYPE_CODES, LIBRARY, SOURCE, Oracle, build, compile_source, load  # noqa: F401
