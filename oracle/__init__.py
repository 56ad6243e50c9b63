"""fp64 CPU oracle for paged-attention decode.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the bench's CPU-baseline
leg, never by the product path.  ``ref`` is the NumPy float64 definition; ``brute`` is a
pure-Python brute force for tiny inputs that pins it.
"""
from . import brute, ref  # noqa: F401
