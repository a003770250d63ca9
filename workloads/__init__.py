"""Seeded synthetic inputs for the DFlash2 draft-block path.

This module is shared by the oracle side and the HIP side and therefore holds
none of the method's arithmetic: only random draws, scaling of those draws to
the stated standard deviations, and the fp32 -> bf16 storage conversion.
"""
from .synth import (  # noqa: F401
    WORKLOADS,
    TENSOR_IDS,
    Shape,
    shape_of,
    bf16_bits,
    bf16_bits_to_f32,
    draw_normal,
    draw_anchor,
    draw_plant_sites,
    make_inputs,
    make_inputs_for,
)
