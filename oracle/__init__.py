"""fp64 CPU oracle of the PACE state path -- TEST INFRASTRUCTURE.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import this
package.  It imports nothing from the library and the library imports nothing from it.
"""
from . import pace_oracle, packing  # noqa: F401
from .packing import LayerCfg  # noqa: F401
