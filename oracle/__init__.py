"""Plain fp64 CPU oracle for one decode step of paged GQA attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product package may import, call or
link anything in this directory; only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, table
or constant generator with the HIP library: every function here is written
from the definition of what the step computes, in float64, with numpy.

Sources cited in this package (the pages are Korean; titles are translated):

* Page A -- 24-ai.news, "vLLM and Tencent Hunyuan upstream two HPC backends
  for NVIDIA Hopper GPUs" (2026-07-06).  Sections used: "Two new HPC backends
  in the vLLM ecosystem" (model shape: 64 query heads, 8 KV heads, head
  dim 128) and "Why does dynamic scheduling matter in attention?" (64-token
  tiles dealt to compute units in proportion to each sequence's current
  length; static split-KV as the baseline; fused RoPE + QK-Norm + KV write;
  BF16 and FP8).
* Page B -- blog.secrett2633.cloud, "[vllm] Introducing the HPC-Ops attention
  backend for high-performance inference in vLLM" (analysis of vLLM PR
  #46020).  Sections used: intro (FP8 E4M3), "Code analysis 2" (RoPE, QK-Norm
  and KV-cache write fused into one kernel; the op writes a caller-provided
  output), "General lessons" (unfused ops repeat memory traffic).
* OCP 8-bit Floating Point Specification (OFP8) rev. 1.0, the E4M3 encoding.

Where the pages are silent the plainest reading is taken; every reading is
listed in the repository's design notes with the same R-number used in the
docstrings here.

Parity status per function (what pins it is in ``tests/test_oracle_*.py``):
every public function is pinned by a library routine, a closed form, an
invariant or brute force, except the choice of RoPE/QK-Norm *order* (R2),
which the pages do not fix: "parity unpinned" for that choice.  The
composition of either order is pinned (an invariant each order alone
satisfies for any weights, and the exact agreement of the two at weight 1).
"""

from .formats import (bf16_bits_to_f64, f64_to_bf16_bits, e4m3_to_f64,
                      f64_to_e4m3, BF16_NAN_BITS, E4M3_NAN_CODE)
from .rope_norm import rope_neox, rms_norm, qk_transform
from .layout import tile_offset, TILE_ELEMS, PAGE_SIZE, HEAD_DIM
from .schedule import (tiles_per_sequence, plan_dynamic, plan_static,
                       default_static_splits, Plan)
from .attention import attend_full, attend_chunk, combine_lse
from .step import (prologue, cache_slot, gather_kv, decode_attention,
                   split_attention, encode_output)
from . import multitoken   # several new tokens per sequence (R20)
from . import qk           # FP8 Q.K^T: q quantised with a per-tensor scale (R23)

__all__ = [
    "bf16_bits_to_f64", "f64_to_bf16_bits", "e4m3_to_f64", "f64_to_e4m3",
    "BF16_NAN_BITS", "E4M3_NAN_CODE", "rope_neox", "rms_norm", "qk_transform",
    "tile_offset", "TILE_ELEMS", "PAGE_SIZE", "HEAD_DIM",
    "tiles_per_sequence", "plan_dynamic", "plan_static",
    "default_static_splits", "Plan", "attend_full", "attend_chunk",
    "combine_lse", "prologue", "cache_slot", "gather_kv", "decode_attention",
    "split_attention", "encode_output", "multitoken", "qk",
]
