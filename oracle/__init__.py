"""CPU oracle for the routed FP4-expert MoE layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library never calls it and
shares no code with it: every FP4 decode, routing decision, grouping step and
product here is written out again, plainly, in float64 numpy.

Each function cites the page passage it follows.  Pages, by title:

* "feat(dsv4): DeepSeek V4 Flash support -- CUDA/VRAM expert tiering, DSML
  tool use, cross-session KV persistence" (PR #1031): the GPU expert path is a
  custom FP4 expert-grouped matvec.
* "DeepSeek V4: the CUDA kernels, as a tier rather than an engine" (PR #772):
  the e8m0 exponent is built from its bit pattern, so s=0 is +0 and s=255 is
  +inf.
* "feat(v4/cuda): the CUDA tier wired into the DeepSeek V4 engine" (PR #1055),
  "What it is": decode runs routed and shared experts in one fused MoE stage;
  prefill routes on the device and runs expert-grouped GEMM rows.
* "Add DeepSeek V4 Flash CPU inference with NVMe expert streaming" (PR #165):
  experts are FP4 E2M1 with UE8M0 scales per group of 32; the 16-entry E2M1
  table is 64 bytes; doubled E2M1 values are integers; six experts per token;
  expert shapes 2048x4096 (gate/up) and 4096x2048 (down); fp64-oracle error
  bounds as the test style; dense tensors are FP8 E4M3 with 128x128 block
  scales (the shared-expert variant, oracle/fp8.py); 43 layers for V4 Flash, run one
  after another in decode (the chained reading of oracle/chain.py).

Every function is pinned by ``tests/test_oracle_pins.py`` against closed
forms, brute force and the printed facts above; none is "parity unpinned".
"""
from .fp4 import E2M1_VALUES, e2m1_value, e8m0_value, dequant
from .fp8 import E4M3_VALUES, Fp8Matrix, e4m3_value, dequant_fp8_block
from .moe import (router_logits, select_experts, group_rows, silu, expert_ffn, dequant_matrix,
                  moe_forward, screen_near_ties)
from .chain import RMS_EPS, rms_norm, f64_to_bf16_bits, norm_input, chain_forward

__all__ = ["E2M1_VALUES", "e2m1_value", "e8m0_value", "dequant", "E4M3_VALUES", "Fp8Matrix",
           "e4m3_value", "dequant_fp8_block", "router_logits", "select_experts", "group_rows", "silu",
           "expert_ffn", "dequant_matrix", "moe_forward", "screen_near_ties", "RMS_EPS", "rms_norm",
           "f64_to_bf16_bits", "norm_input", "chain_forward"]
