"""CPU oracle of the In-Place TTT gated-MLP prefill (test infrastructure only:
used by the tests, the smoke check and the benchmark's CPU baseline)."""
from .ttt_oracle import *  # noqa: F401,F403
