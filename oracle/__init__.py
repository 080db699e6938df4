"""Test infrastructure: the fp64 CPU oracle and the integer schedule reference.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package.  The HIP library never does, and this package never imports the
library.
"""
