"""CPU oracle (fp64, dense Sylvester H) -- test infrastructure only.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg import
this package; the product path never does.
"""
from .qwha_oracle import *  # noqa: F401,F403
from .qwha_oracle import __all__  # noqa: F401
