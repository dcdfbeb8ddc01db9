"""CPU oracle for the NVFP4 linear layer -- test infrastructure only.

Only tests/, __graft_entry__.smoke() and bench.py's CPU-baseline leg may
import this package.  The product library never does.
"""
