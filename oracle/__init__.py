"""fp64 CPU oracle (test infrastructure only; never on the product path)."""
from .lazyflash_oracle import *  # noqa: F401,F403
from .lazyflash_oracle import __all__  # noqa: F401
