"""CPU oracle for the top-1 MoE gate (test infrastructure only).

Only tests/, the smoke check in __graft_entry__ and the CPU-baseline leg of
bench.py may import this package.  The HIP library and its Python binding never
do.
"""
from . import moe_oracle, brute  # noqa: F401
