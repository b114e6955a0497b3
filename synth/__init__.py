"""Seeded synthetic inputs for the depth-routing read (AttnRes / MHAR / LR-AttnRes).

This package holds input generation only: workload shapes, the site schedule
(which bank rows each routing site reads), the random draws and the rounding of
drawn values to the storage dtype.  None of the routing arithmetic lives here,
so both the CPU oracle and the HIP path can take their inputs from it without
sharing any of the method's computation.
"""

from .workloads import (  # noqa: F401
    WORKLOADS,
    Workload,
    block_schedule,
    full_schedule,
    get_workload,
    read_schedule,
)
from .draws import Inputs, bf16_bits, bf16_round, sample_tokens  # noqa: F401
from .delta import DELTA_SHAPES, DeltaInputs, DeltaShape  # noqa: F401
from .lists import LIST_SHAPES, ListInputs, ListShape  # noqa: F401
from .blocks import BLOCK_SHAPES, BlockInputs, BlockShape  # noqa: F401
