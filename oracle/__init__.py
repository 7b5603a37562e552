"""fp64 CPU oracle for the routed MoE FFN (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this package.  See moe_oracle.py for what it computes and its sources.
"""
