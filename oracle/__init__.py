"""fp64 CPU oracle of the block-diffusion refinement step.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or execute anything
under ``oracle/``.  The HIP product path never does, and this package imports
nothing from it.
"""
from .refine import *  # noqa: F401,F403
