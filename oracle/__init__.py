"""CPU oracle (test infrastructure only): the plain fp64 definition of the
depth-routing read, its backward and the site schedule.  Imported only by the
tests, the smoke check and the benchmark's CPU-baseline leg."""

from .attnres_oracle import (  # noqa: F401
    EPS,
    block_reads,
    delta_backward,
    delta_forward,
    inv_rms,
    key_slice,
    route_backward,
    route_forward,
    run_block_routing,
    run_schedule,
    source_inv_rms,
)
