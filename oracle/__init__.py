"""CPU oracle of the W4A16 mixture-of-experts expert layer (test infrastructure).

This package is a plain, slow, float64 reference of what the layer computes.
It exists to check the HIP library and must never be part of it: only the
tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  It shares no code with the HIP path and imports
nothing from it.

Sources (the four pages the method is described on):

* "sglang PR 31552" summary on prhub.com.cn: Marlin MoE W4A16 kernel; its
  unit test ``test_fused_marlin_moe_large_non_ep_schedule`` holds the
  per-expert reference loop and the bias placement.
* "sglang PR 28231" summary on prhub.com.cn: MXFP4 MoE on Marlin; the gate/up
  de-interleave (``deinterleave_moe_mxfp4_w13_for_marlin``) and the
  GPT-OSS activation (``swiglu_gpt_oss_sigmoid_alpha_contiguous``).
* "013-moe-middle-tiles.py" (bishal.us open-kernel-challenge experiment): the
  NVFP4 expert slice, ``expert_map`` routing, ``moe_align_block_size``, the
  two GEMMs, ``silu_and_mul`` and the post-expert-norm weighted sum
  (``_expert_norm_factors`` / ``_expert_norm_sum``).
* "sglang PR 35760" summary on prhub.com.cn: the W4AFP8 per-token -> per-tensor
  float8 requant of the dispatched activations (``oracle/requant.py``).

Every function pinned by a test says what pins it; see ``tests/test_oracle*.py``.
"""
from .formats import (E2M1_VALUES, decode_bf16, decode_e2m1, decode_e4m3fn, decode_e8m0,
                      decode_uint4b8, round_to_bf16, bf16_bits_of)
from .moe import (route_local, align_capacity, moe_align, dequant, split_gate_up,
                  act_silu_mul, act_swiglu_alpha, expert_forward, combine, moe_layer,
                  norm_weight)

__all__ = [
    "E2M1_VALUES", "decode_bf16", "decode_e2m1", "decode_e4m3fn", "decode_e8m0",
    "decode_uint4b8", "round_to_bf16", "bf16_bits_of", "route_local", "align_capacity",
    "moe_align", "dequant", "split_gate_up", "act_silu_mul", "act_swiglu_alpha",
    "expert_forward", "combine", "moe_layer", "norm_weight",
]
