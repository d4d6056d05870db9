"""Float64 CPU oracle of the LFM3-1.7B hybrid decoder forward pass.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports this package: only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may use it. It shares no
code with the HIP library (it parses the weight blob with its own reader) and it is deliberately
plain and slow: numpy float64, no blocking or fusion beyond what the definitions state.

Every function cites the passage of the pages it follows. Page names used in citations:
- "LFM3-1.7B port" = the Core AI knowledge note on porting LFM3-1.7B (comparison table, the
  "window_size, with no mask input" section, the "partial_rotary_factor" section, the fp32-gate
  paragraph, "Chunked prefill" and "--pad-tail").
- "TensorFold #1491" = the issue adding native Metal support for the LFM3 MLX checkpoints.
- "TensorFold PR #1508" = the pull request serving LFM3-1.7B NVFP4 on CUDA (both heads).

Parity status of each part is listed in ``oracle/ref.py``'s module docstring.
"""
from .ref import (  # noqa: F401
    Blob, Oracle, SlotState, dequant, unpack_codes, rmsnorm, rope_angles, rope_apply, silu, sigmoid,
    attention_rows, attention_core, conv_step, e2m1_values, e4m3_values, dequant_nvfp4,
    dequant_fp8_block, load_weight, greedy_argmax, bf16_round, f16_round, top2_margin,
)
