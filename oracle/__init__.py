"""CPU fp64 oracle of the recurrent-block forward.

TEST INFRASTRUCTURE: imported only by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py.  The HIP path neither imports nor calls it.
"""
