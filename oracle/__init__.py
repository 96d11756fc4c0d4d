"""CPU oracle of the stage decoder forward -- test infrastructure only.

Importable by ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg.
The GPU path never imports it, and it never imports the GPU path.
"""
from .decoder import *  # noqa: F401,F403
