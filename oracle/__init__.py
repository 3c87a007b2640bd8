"""CPU oracle for the MoE routing-and-balancing layer.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously-correct
reference (fp64 floats, Python integers) that the GPU path is checked against.
Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import it; the GPU library never calls into it and shares no
code with it.
"""
from .moe_oracle import *  # noqa: F401,F403
