"""CPU oracle for paged decode attention — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and its
Python binding) never imports, links or calls it, and it imports nothing from the
product path.
"""

from .oracle import *  # noqa: F401,F403
from .block_manager import BlockManager, OutOfBlocks, move_requests  # noqa: F401
