"""CPU oracle for the UFP4 hot path -- test infrastructure only.

Only the tests, the smoke check and the bench's CPU-baseline leg may import
this package.  The product path (the HIP library and its Python binding) never
does.
"""
from . import ufp4_oracle  # noqa: F401
