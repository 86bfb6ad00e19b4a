"""CPU oracle of the grouped, weight-quantized MoE FFN (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library never does, and this
package never imports the GPU library.
"""
from .moe_oracle import *  # noqa: F401,F403
