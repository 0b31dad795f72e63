"""Seeded synthetic inputs for the DSA hot path.

This module only draws random tensors and lays them out; it computes none of
the method's steps.  Both the GPU library's tests/benchmark and the CPU
oracle's tests consume what it produces.

Recipe (every tensor has its own generator, seeded ``1000 * cfg + tensor_id``,
so adding a tensor never shifts the others):

* indexer q / k: N(0, 1) in fp32, one scale per token = amax / 448 over the
  token's values, codes = torch's float32 -> float8_e4m3fn cast of x / scale
  (OCP E4M3, round to nearest even);
* indexer per-head weights: N(0, 1 / H_I) fp32;
* MLA q and latent KV rows: N(0, 1) fp32 rounded to bf16;
* page layouts: seeded random permutations (identity where a config asks for
  contiguous storage);
* the exact-arithmetic set "E1": integer FP8 codes in [-4, 4], power-of-two
  scales and weights that are multiples of 1/16 in [-1, 1].
"""
from .gen import (  # noqa: F401
    gen, normal, bf16_normal, fp8_per_token, randperm, e1_codes, e1_pow2_scales, e1_weights,
    bf16_bits, fp8_bits,
)
from .configs import CONFIGS, PrefillInputs, DecodeInputs, make_prefill, make_decode, decode_queries  # noqa: F401
