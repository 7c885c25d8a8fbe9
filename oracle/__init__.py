"""CPU oracle for the int6 / int5 / int8 per-row scoring pass, its export side
and the forward-only quantisation-aware weights.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything here.  The HIP
library never does, and this package imports nothing from it.

It is a plain, slow, obviously correct restatement of what the scoring pass
computes, written from these web pages (cited by page and section):

* pwwt.cn, "parameter-golf 16MB 极限压缩实战：11L MLP3x + Int6 QAT + zstd-22
  记录详解" -- sections 架构：11 层 U-Net 变压器 (model), 训练时的模拟量化 and
  后训练量化导出 (row quantiser), 滑动窗口评估 (sliding-window eval).
* kwkr.cn write-up of parameter-golf PR #363 "Depth Recurrence +
  Mixed-Precision Quantization" -- Middle-Cycle Stem/Core/Tail layout,
  DepthLoRA, BigramHash, and the Noisy-QAT code block (the 1e-12 amax floor).
* pigsec.cn mirror of the openai/parameter-golf README -- bits-per-byte as the
  tokenizer-agnostic score; parallel residual lanes and the looped layers
  4-5 of later records.

Modules:
  ``quant``   -- row quantiser, step by step in IEEE binary32 (bit-exact gate).
  ``model``   -- the transformer forward in float64 with dequantised weights.
  ``windows`` -- the sliding-window plan and bits-per-byte.
  ``export``  -- int6 / int5 bit packing, code histogram and entropy,
                 artifact bytes, dequantisation to fp32 / bf16.
  ``qat``     -- STE fake quantisation, Noisy-QAT noise, Philox4x32-10.

Every function here is pinned by CPU tests in ``tests/test_oracle_*.py``
against closed forms, brute force, invariants and the pages' printed numbers.
"""
from . import quant, model, windows, export, qat  # noqa: F401
from .quant import quantize_rows, quantize_model  # noqa: F401
from .windows import plan_windows, score, bpb  # noqa: F401
