"""CPU oracle (test infrastructure only): a plain, slow reference of the sketch path.

Only tests/, the smoke check and the benchmark's CPU-baseline leg may import it.
"""
from .rgc_oracle import *  # noqa: F401,F403
