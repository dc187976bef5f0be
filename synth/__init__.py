"""Seeded synthetic inputs for the SmoothQuant W8A8 linear workloads.

This package only draws random numbers and casts them to the storage dtype of
each workload. It holds none of the method's arithmetic, so both the CPU
oracle and the HIP path can consume its tensors.
"""
from .workloads import (  # noqa: F401
    WORKLOADS,
    Site,
    Workload,
    site_inputs,
    token_block,
    calibration_block,
    weight_block,
    outlier_channels,
    to_numpy,
    rand_tokens,
    rand_int8,
    rand_positive,
    norm_params,
)
