"""CPU oracle for RecSA -- test infrastructure only (see recsa_oracle)."""
from .recsa_oracle import *  # noqa: F401,F403
