"""CPU oracle of the RLT decoder transition, of its backward pass, and of the encoder and
readout/sampler around it.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the package smoke check and by the
benchmark's CPU-baseline leg, never by the product path.
"""
from .rlt_oracle import *  # noqa: F401,F403
from .rlt_oracle import __all__ as _fwd
from .rlt_backward import *  # noqa: F401,F403
from .rlt_backward import __all__ as _bwd
from .rlt_head import *  # noqa: F401,F403
from .rlt_head import __all__ as _head

__all__ = list(_fwd) + list(_bwd) + list(_head)
