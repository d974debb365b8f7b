"""CPU oracle for the block-scaled FP4 routed-MoE FFN layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this package:
only the test-suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` may use it.  It shares no code, tables or helpers with the HIP
library under ``block_scaled_fp4_sqrtsoftplus_amd/``; the two only see the same
seeded inputs from ``synth``.

The oracle is a plain, slow, step-by-step NumPy implementation of what the
layer computes, in float64 unless a step fixes another precision.  Sources:

* "DeepSeek-V4-Flash-SI" model card, section 架构特性: the MoE paragraph
  (256 routed + 1 shared expert, top-6, sqrtsoftplus scoring, hash routing in
  the first layers, routing scale 1.5, SwiGLU clamp +-10) and the 低精度计算
  paragraph (FP4 E2M1 expert weights with one F8_E8M0 scale per 32 elements,
  activations quantized online to FP8 E4M3 per 128 elements with a
  power-of-two scale).
* same card, section 模型训练 table: activation quantization is dynamic FP8
  E4M3 with a ue8m0 scale.
* "DeepSeek-V4-Pro-0813-nvfp4-DSpark" article, sections 阶段三导出 (the
  MXFP4 vs NVFP4 storage table: same E2M1 nibble grid, per-32 E8M0 vs per-16
  E4M3 scales) and "关于 MXFP4 的无损种子" (an E2M1 -> E4M3 cast that splits
  each byte into its two nibbles, decodes them through the FP4 table and
  rewrites the scale per 128-block).
* "DeepSeek-V4-Flash-0731-W4AFP8-mt" card, section 权重约定: expert weights
  stored [N, K/2] (two 4-bit values per byte) with a [N, K/groups] scale.

Modules:
  formats  - E2M1 / E8M0 / E4M3 / bf16 codecs
  quant    - per-128 activation quant, MXFP4 dequant, NVFP4 and E4M3 re-expressions
  route    - router logits, sqrtsoftplus, top-k, hash routing, permutation
  ffn      - routed expert FFN, shared expert, combine, whole layer

Parity status: every function is pinned by tests under tests/test_oracle_*.py
(closed forms, brute force, library routines, invariants the pages state).
Against the real model the layer is parity unpinned: no checkpoint,
activation dump or printed worked example exists for it.
"""

from . import formats, quant, route, ffn  # noqa: F401
