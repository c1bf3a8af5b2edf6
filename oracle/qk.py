"""Q.K^T arithmetic with an FP8 cache (reading R23), in fp64.

Page A, "Why does dynamic scheduling matter in attention?", offers BF16 and
FP8 backends, and page B's intro names E4M3 as the FP8 type; the pages do not
say how q enters an FP8 product.  The plainest reading that mirrors the
cache's per-tensor scales (R9): q is quantised with a caller-given per-tensor
q_scale, code = RNE(clamp(q * r, -448, 448)), where r is 1/q_scale rounded to
fp32 and the product q * r is rounded to fp32 first (so both sides take the
integer decision on the same fp32 value).  The scores are then those of the
decoded q, code * q_scale; everything after the scores is unchanged.

Test infrastructure: only tests, smoke() and the benchmark's CPU baseline use
the oracle.
"""

import numpy as np

from .formats import bf16_bits_to_f64, e4m3_to_f64, f64_to_e4m3


def quantize_query(q_bits, q_scale):
    """E4M3 codes of BF16 queries (bit patterns) under R23."""
    inv = np.float32(1.0) / np.float32(q_scale)
    x = bf16_bits_to_f64(q_bits).astype(np.float32) * inv      # one fp32 rounding
    return f64_to_e4m3(x.astype(np.float64))


def query_values(q_bits, cfg):
    """The query values the scores use: the BF16 values, or (cfg["qk_dtype"] ==
    "fp8") the decoded E4M3 codes times q_scale."""
    if cfg.get("qk_dtype", "bf16") == "bf16":
        return bf16_bits_to_f64(q_bits)
    q_scale = float(np.float32(cfg["q_scale"]))
    return e4m3_to_f64(quantize_query(q_bits, q_scale)) * q_scale
