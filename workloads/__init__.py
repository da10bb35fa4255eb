"""Seeded synthetic inputs shared by the CPU oracle's tests, the GPU tests and
the benchmark.  Holds input generation only, none of the attention arithmetic."""
from .generate import (BLOCK_SIZE, BASE_SEED, SeqGroup, Workload, f32_to_bf16_bits, make_config,
                       make_decode, make_prefill, config0, config1, config2, config3, config4,
                       permute_block_ids, unshare_blocks, lens_config1, lens_config2,
                       lens_config3, storage_dtype, nan_fill, CONFIGS, fp8_codes, fp8_pools,
                       FP8_NAN_CODE, sampler_inputs, SAMPLER_PARAMS)

__all__ = [
    "BLOCK_SIZE", "BASE_SEED", "SeqGroup", "Workload", "f32_to_bf16_bits", "make_config",
    "make_decode", "make_prefill", "config0", "config1", "config2", "config3", "config4",
    "permute_block_ids", "unshare_blocks", "lens_config1", "lens_config2", "lens_config3",
    "storage_dtype", "nan_fill", "CONFIGS", "fp8_codes", "fp8_pools", "FP8_NAN_CODE",
    "sampler_inputs", "SAMPLER_PARAMS",
]
