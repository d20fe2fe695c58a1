"""CPU oracle for the fused MoE expert FFN.

TEST INFRASTRUCTURE ONLY. Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this
package. The product path (the HIP library and its Python binding) never
routes through it and shares no code with it.
"""
from .moe_oracle import *  # noqa: F401,F403
