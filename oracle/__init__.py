"""CPU oracle of the DSA hot path -- test infrastructure only.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this package.  The library in sparse_attention_15_amd/ never does.
"""
from . import dsa_oracle  # noqa: F401
