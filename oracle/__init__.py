"""CPU oracle for the SVDQuant W4A4 linear layer (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this package; the GPU library never does.
"""
from .svdq_oracle import *  # noqa: F401,F403
from .svdq_oracle import INT4_GROUP, FP4_BLOCK, E2M1_GRID  # noqa: F401
from .awq_oracle import *  # noqa: F401,F403
from .gelu_oracle import *  # noqa: F401,F403
from .rsvd_oracle import *  # noqa: F401,F403
from .qkv_oracle import *  # noqa: F401,F403
from .nvfp4_oracle import *  # noqa: F401,F403
