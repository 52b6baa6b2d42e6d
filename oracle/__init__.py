"""CPU oracle (test infrastructure only; see forcing_kv.py).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may use it.
"""
