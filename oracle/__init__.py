"""Oracle package: TEST INFRASTRUCTURE ONLY (tests, smoke check, CPU baseline).

The product path never imports this package.
"""
from .beam_oracle import *  # noqa: F401,F403
from .beam_oracle import __all__  # noqa: F401
