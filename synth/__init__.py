"""Seeded synthetic inputs shared by the oracle tests and the HIP path.

This package only draws random numbers and rounds them to the storage dtype.
It contains none of the compression or decode arithmetic.
"""
from .kvgen import CONFIGS, Workload, make_workload, config_by_name, gaussian  # noqa: F401
