"""CPU oracle for fine-grained FP8 quantization and block-scaled FP8 GEMMs.

TEST INFRASTRUCTURE ONLY. This package is the slow, plain, obviously-correct
definition that the HIP library is checked against. Only the test suite, the
smoke check in ``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py``
may import it. The product path (``fp8_block_scaled_quant_amd``) never imports,
links or calls anything here, and this package never imports the product path:
the two share no code, no tables and no helpers.

Everything is numpy on the CPU. Floating-point work that is not fixed by a
format (fp32 division for scales and scaled values, bf16 rounding) is done in
the precision the definition names; dequantized GEMMs are accumulated in fp64.

Sources (the web pages this method is described on), cited by title and
section throughout:

* [SkyRL-FP8]  "Anyscale、SkyRL で FP8 学習・ロールアウトをサポートし一貫性を維持"
  (news.ainew.jp translation of the Anyscale/SkyRL article on FP8 training and
  rollout with on-policy weight sync).
* [AIS]        "AIS: Adaptive Importance Sampling for Quantized RL" explainer
  (kasblo.com): FP8 format table and the symmetric quantizer equation.
* [Jet-RL]     "Jet-RL: Enabling On-Policy FP8 Reinforcement Learning with
  Unified Training and Rollout Precision Flow" (gist.science summary):
  quantization scheme (1x128 activations, 128x128 weights, 1x128/128x1 WGrad).

Parity status of each function is stated in its docstring ("pinned by ..." or
"parity unpinned").
"""

from . import fp8_formats, quantize, gemm, weight_sync, producers, fp8_param  # noqa: F401
