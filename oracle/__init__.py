"""CPU oracle (test infrastructure only; see pa_oracle.py).

Only the tests, the entry script's smoke check and the bench's CPU-baseline
leg may import this package. The product path never does.
"""
from .pa_oracle import *  # noqa: F401,F403
