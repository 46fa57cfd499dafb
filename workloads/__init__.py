"""Seeded synthetic inputs for paged-KV decode.

This package is shared by the tests, the benchmark and the smoke check. It
draws random numbers and lays them out in the paged-cache format. It holds
none of the attention arithmetic: neither the HIP path nor the CPU oracle
lives here, and nothing here imports either of them.
"""

from .paged_decode import (  # noqa: F401
    CONFIGS,
    VARIANT_CONFIGS,
    DecodeCase,
    WorkloadConfig,
    fp8_quantise_per_token,
    make_case,
    make_config_case,
    permute_pool,
    repage,
)
