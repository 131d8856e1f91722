"""Seeded synthetic inputs for block-sparse attention requests.

Shared by the tests, the benchmark and the oracle checks.  This module draws
random numbers and builds masks with the structure of the workloads the Tessera
paper evaluates (video-diffusion masks at 9-12% mean density, section 7.1);
it contains none of the attention arithmetic.
"""

from .gen import (  # noqa: F401
    CONFIGS,
    GEOMETRIES_C5,
    config,
    mask_clustered,
    mask_iid_diag,
    mask_spatiotemporal,
    qkv,
    request_c5,
)
