"""fp64 CPU oracle for the Shampoo optimizer step -- test infrastructure only.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package.  The GPU library (second_order_optimizer_amd) never imports it,
and the two share no code.
"""
from .shampoo_oracle import *  # noqa: F401,F403
