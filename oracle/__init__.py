"""CPU oracle for the top-k token-choice MoE-layer forward.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or links
this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, constants or
helpers with the HIP library.

See ``oracle/moe_oracle.py`` for the computation and its citations.
"""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import __all__  # noqa: F401
