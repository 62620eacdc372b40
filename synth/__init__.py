"""Seeded synthetic inputs for the CSA/HCA path.

This module is shared by the tests, the benchmark and the smoke check.  It holds none of the
method's arithmetic: it only draws random numbers (numpy PCG64) and packs them into the
storage formats the boundary takes.

* bf16 tensors: float32 normal draws truncated to their upper 16 bits (truncation, not the
  method's round-to-nearest-even, so no rounding code is shared with either side).
* E4M3 tensors: codes are assembled from bit fields - sign and binary exponent taken from a
  normal draw, mantissa bits uniform - so the code magnitudes follow N(0,1) to within a
  binade; exponent fields stay in 0..14, so no NaN code is ever produced.
* the RoPE inverse-frequency table base^(-2i/r) is a configuration input of the layer.
"""
from .inputs import (WORKLOADS, Workload, bf16_normal, e4m3_normalish, rope_inv_freq,
                     weight_cols, tail_shape, layer_inputs, decode_cache_inputs)

__all__ = ["WORKLOADS", "Workload", "bf16_normal", "e4m3_normalish", "rope_inv_freq",
           "weight_cols", "tail_shape", "layer_inputs", "decode_cache_inputs"]
