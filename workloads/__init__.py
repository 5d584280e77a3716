"""Seeded synthetic inputs shared by the HIP path's tests, the oracle's tests
and the benchmark.  Holds no part of the method's arithmetic."""
from .synth import (  # noqa: F401
    CONFIG_ORDER, PRESETS, STAGE_DEPTHS, TAU, Workload, Zipf, envelope,
    f32_to_bf16_bits, make, make_from_spec, plant_path, rope_table, sampling_uniforms,
    workload_rope_table,
)
