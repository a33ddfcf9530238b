"""CPU oracle for the MM-DiT block hot path (test infrastructure only).

Only tests, the smoke check and the benchmark's CPU-baseline leg import this
package; the product path never does.
"""
from .mmdit_oracle import *  # noqa: F401,F403
from . import mmdit_oracle  # noqa: F401
