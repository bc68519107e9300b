"""CPU oracle for batch-1 Llama decode — TEST INFRASTRUCTURE, not part of the product path.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import, call or execute anything in this package. The HIP decode library never
routes through it and shares no code with it: the two meet only in the seeded input
generator module ``workloads``, which holds no decode arithmetic.

What it computes. The decode-megakernel pages (AutoMegaKernel paper index, Abstract;
gist.science explainer, Technical Summary > Problem Statement and Methodology) compile
the forward pass of a HuggingFace Llama-family model into one kernel per decoded token
and claim it reproduces eager HuggingFace greedy decode. The method therefore reaches
exactly (up to rounding order) the ordinary Llama decode step, and this oracle is that
definition written out in plain NumPy float32 (the precision the workload fixes for the
oracle), one operation at a time, plus the W8A16 weight transform (Key Contributions:
int8 weight-only quantized megakernels).

Modules:
  numerics  — bf16 <-> fp32 bit conversions (round-to-nearest-even)
  quant     — symmetric per-output-row int8 quantizer
  llama     — RMSNorm, RoPE, GEMV, GQA attention, SwiGLU, the decode step, and an
              independently written full-sequence causal forward used as a cross-check

Pins: every function is checked by ``tests/test_oracle_*.py`` against closed forms,
invariants, brute force and hand-derived cases. The whole-model logits at the real
shapes are pinned only through those parts (no checkpoint or printed logits exist):
parity unpinned externally for the composed model, see the test docstrings.
"""
from .numerics import bf16_bits_to_f32, f32_to_bf16_bits, round_bf16  # noqa: F401
from .quant import quantize_rows_int8, dequantize_rows  # noqa: F401
from .llama import OracleModel, rmsnorm, rope_tables, apply_rope, gemv, attention_head, silu  # noqa: F401
