"""CPU oracle (test infrastructure only; see sparse_ffn_oracle)."""
from .sparse_ffn_oracle import *  # noqa: F401,F403
from .sparse_ffn_oracle import __all__  # noqa: F401
