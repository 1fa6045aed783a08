"""CPU oracle for fine-grained FP8 (E4M3) quantization and block-scaled FP8 GEMMs.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it. It is a plain, slow, obviously-correct numpy
implementation written from the pages' statement of the method, and it shares
no code, tables or constants with the HIP library.

Sources (cited by page title and paragraph/section; the pages are the
DeepSeek-V3 FP8 material collected for this method):

* dssusan.co.kr FP8 excerpt (untitled board post), paragraphs 1-4:
  online max-abs per 1x128 activation tile and 128x128 weight block,
  integral power-of-2 scales, per-group scales along the inner dimension K,
  FP32 promotion of MMA partials, 1x128 -> 128x1 conversion for backward.
* "Deepseek - Not For everyone", paragraphs 3-4: max-abs is scaled to the
  largest representable FP8 value; scales are multiplied in as dequantization.
* youlimart.com FP8 excerpt, paragraphs 1-3: tile/block groupings; Fprop,
  Dgrad and Wgrad all in FP8; GEMMs take FP8 inputs and write BF16 or FP32.
* "FP8 mixed precision - где и как DeepSeek снизили точность вычислений?",
  sections on fine-grained quantization, FP32 accumulation, and E4M3 for all
  three GEMMs.

Modules:
    e4m3   -- OCP E4M3FN decode/encode (all pinned).
    quant  -- 1x128, 128x1 and 128x128 quantizers, max-abs and pow2 modes, and the
              FP8 -> FP8 1x128 -> 128x1 re-quantization (all pinned).
    gemm   -- block-scaled GEMM reference for Fprop/Dgrad/Wgrad and the grouped
              variant, plus output rounding to FP32/BF16 (all pinned).
    study  -- quantization-error study of the scaling rules (per-tensor,
              1x128, 128x128, power-of-2, delayed), built on the pinned
              quantizers; ``python -m oracle.study`` prints the table.
"""

from . import e4m3, quant, gemm  # noqa: F401
