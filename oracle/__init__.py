"""CPU oracle for 4-bit weight-only GEMM (TEST INFRASTRUCTURE ONLY).

Plain, slow, obviously-correct numpy definitions of what the fused
dequantize-and-multiply path computes.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import this package; the product library under ``bit_weight_only_gemm_amd``
never does, and shares no code, table or constant generator with it.

Sources (cited by page title and section throughout):

[P1] "GPTQ、AWQ与Bitsandbytes：大模型量化三大技术路径深度对比" (tqpw.cn/news/80721)
[P2] "模型量化实践：GPTQ 与 AWQ 在生产环境的精度与速度权衡" (jsqmd.com/news/975148)
[P3] "LLM 量化技术详解：GPTQ、AWQ 与 GGUF 的选型与实践"
     (cloud.tencent.com/developer/article/2726413)
[P4] "GPTQ与bitsandbytes对比：谁是2024年大模型量化的终极选择？"
     (blog.csdn.net/gitblog_00436/article/details/141051550)
[P5] "LLM量化技术深度对比:GPTQ vs AWQ vs bitsandbytes 2026基准全解析"
     (5ulink.com/archives/1952)

Modules
-------
fp     -- IEEE rounding helpers (fp32 -> bf16 round-to-nearest-even by bit ops).
int4   -- RTN group quantizer, GPTQ-style packing/unpacking, int4 dequant.
intb   -- the same at 3, 4 or 8 bits (bit-stream packing of 32-code runs).
nf4    -- NF4 codebook (closed form), block quantizer, double quant, dequant.
gemm   -- fp64 reference product and the relative-error score.
repack -- reference implementation of the repacked tile layout and its inverse.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against closed forms, brute force, exact rational arithmetic or independent
library routines.  Bit-compatibility with third-party checkpoints or libraries
is "parity unpinned": the pages give no byte layout for them.
"""

from . import fp, int4, intb, nf4, gemm, repack  # noqa: F401
