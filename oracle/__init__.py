"""Reference oracle (test infrastructure only; see oracle.oracle)."""
from .oracle import *  # noqa: F401,F403
from .oracle import QK, fp16_bits_to_f64  # noqa: F401
