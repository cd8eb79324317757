"""CPU oracle (test infrastructure only; the product package never imports it)."""
from .nvfp4_oracle import *  # noqa: F401,F403
from . import nvfp4_oracle  # noqa: F401
