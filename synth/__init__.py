"""Seeded synthetic inputs for the selective scan (S6) and its one-token decode step.

This module only draws numbers: it holds none of the scan's arithmetic. Both the
fp64 oracle (``oracle/``) and the HIP library (``selective_state_space_06_amd``)
are fed from here, so they see bit-identical inputs.
"""
from .inputs import (  # noqa: F401
    CONFIGS,
    ScanInputs,
    DecodeInputs,
    round_to_bf16,
    scan_inputs,
    decode_inputs,
    sample_rows,
    SSD_CONFIGS,
    SSDInputs,
    ssd_inputs,
)
