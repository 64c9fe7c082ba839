"""CPU oracle of the weight-only low-bit linear layer (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package; the HIP library and its Python binding never do."""
from .reference import *  # noqa: F401,F403
from . import reference  # noqa: F401
