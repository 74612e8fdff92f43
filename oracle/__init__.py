"""Plain CPU oracle for the block-scaled FP8 / NVFP4-style linear path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product (the HIP library and its
Python binding) imports, links or calls this package; only ``tests/``, the
smoke check in ``__graft_entry__`` and the CPU-baseline leg of ``bench.py``
do.  It shares no code, tables or constants generator with the GPU path.

Everything is written from the definitions on the pages (and, for the bit
layouts the pages only name, from the public OCP format specifications), in
numpy with fp64 arithmetic wherever the pages do not fix a precision:

* ``formats`` -- E4M3FN / E8M0 / E2M1 / BF16 codecs.
* ``quant``   -- 1x128 activation and 128x128 weight FP8 quantization with
  fp32 or UE8M0 scales.
* ``gemm``    -- block-scaled FP8 GEMM (dense and MoE-grouped), fp64
  accumulation of dequantized operands.
* ``fp4``     -- NVFP4-style quantization (e2m1 codes, 16-element e4m3 group
  scales, fp32 tensor scale) and its GEMM.

Page citations use the page titles:
  [FG-FP8]  "Transformers 中的细粒度 FP8 量化：配置、DeepGEMM 加速路径与 UE8M0
            缩放格式完全指南" (sections 一 .. 九)
  [HF-PT]   "FP8 de granularidade fina" (Transformers docs, Portuguese)
  [NVFP4]   "混合精度策略解析：NVIDIA Mistral-Medium-3.5-128B-NVFP4中FP8与NVFP4的协同工作"
Format layouts: [OFP8] OCP 8-bit Floating Point Specification v1.0;
[MX] OCP Microscaling Formats (MX) Specification v1.0.

Where the pages leave a step open, the reading taken is stated in the
docstring of the function that takes it.
"""

from . import formats, quant, gemm, fp4  # noqa: F401
