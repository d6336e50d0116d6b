"""fp64 CPU oracle for PBSA -- test infrastructure only (tests, smoke check, CPU baseline)."""
from .pbsa_oracle import *  # noqa: F401,F403
