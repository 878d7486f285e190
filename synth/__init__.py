"""Seeded synthetic inputs for paged MLA decode.

This module only draws random numbers and lays them out (sequence lengths,
block tables, query and cache values, sparse index lists).  It holds none of
the attention arithmetic, so both the FP64 oracle's tests and the HIP path's
tests and benchmark can take their inputs from it.
"""
from .configs import WORKLOADS, make_config, make_case, bf16_from_f32

__all__ = ["WORKLOADS", "make_config", "make_case", "bf16_from_f32"]
