"""Oracle for the MSA routing + sparse-attention path: TEST INFRASTRUCTURE ONLY.

Imported by tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg;
never by the product package.  See msa_oracle.py for the readings it encodes.
"""
from . import msa_oracle, bruteforce  # noqa: F401
