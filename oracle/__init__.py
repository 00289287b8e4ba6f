"""fp64 CPU oracle for MLA decode (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package.  It shares no code with the HIP path.
"""
from . import mla_oracle

__all__ = ["mla_oracle"]
