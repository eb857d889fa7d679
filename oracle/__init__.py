"""fp64 CPU oracle -- test infrastructure only (see lrc_oracle for the header)."""
from .lrc_oracle import *  # noqa: F401,F403
from .lrc_oracle import __all__  # noqa: F401
