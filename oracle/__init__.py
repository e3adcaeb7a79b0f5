"""CPU oracle package -- TEST INFRASTRUCTURE ONLY (tests, smoke check, benchmark CPU baseline).
The library's product path never imports it."""
from .csa2_oracle import *  # noqa: F401,F403
