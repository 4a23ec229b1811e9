"""CPU oracle for the TokenGate gated-prefill path (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  The library never does; its product path runs
entirely in the HIP kernels of ``libtokengate.so``.
"""
from .tokengate_oracle import *  # noqa: F401,F403
from .tokengate_oracle import __all__  # noqa: F401
