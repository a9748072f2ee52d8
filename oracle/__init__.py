"""fp64 CPU oracle of the rotated-basis matrix-optimizer step.

TEST INFRASTRUCTURE: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it. The product path (the HIP
library and its Python binding) never imports or calls anything here.
"""

from .rotated_adam import *  # noqa: F401,F403
from .rotated_adam import __all__  # noqa: F401
