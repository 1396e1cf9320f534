"""Seeded synthetic input generators shared by the oracle tests, the GPU
parity tests and the benchmark. Holds no attention arithmetic."""
from .gen import (CONFIGS, D_QK, D_V, MERGE_TOKENS, PAGE_SIZE, SOFTMAX_SCALE, AppendInputs,
                  MergeInputs, Workload, f32_to_bf16_bits, f32_to_e4m3_bits, make_append_inputs,
                  make_config, make_merge_inputs, make_workload,
                  plant_rising_keys)
