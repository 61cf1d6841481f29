"""FP64 CPU oracle (test infrastructure only; see muse_oracle's header)."""
from .muse_oracle import *  # noqa: F401,F403
from .muse_oracle import __all__  # noqa: F401
