"""CPU oracle of the FlashMap draft-step attention path (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline leg
may import it.  The product path (the HIP library and its binding) never does.
"""

from .fm_oracle import *  # noqa: F401,F403
from .fm_oracle import __all__  # noqa: F401
