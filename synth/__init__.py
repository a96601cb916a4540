"""Seeded synthetic inputs shaped like the video-DiT attention workloads.

This package only draws inputs: token grids, Q/K/V tensors, block masks and the
random start block of the subspace iteration.  It contains none of the
arithmetic of the attention or reordering method, and it is shared by the
tests, the benchmark and the smoke check so that the oracle and the HIP path
see identical inputs.
"""

from .workloads import (  # noqa: F401
    CONFIGS,
    Workload,
    WorkloadConfig,
    drift_states,
    get_config,
    make_workload,
    minhash_params,
    random_tiny_case,
    wide_range_case,
)
from .hilbert import gilbert2d, gilbert3d, video_hilbert_order  # noqa: F401
