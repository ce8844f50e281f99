"""Plain, slow CPU oracle for the NF4 + double-quant QLoRA linear layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (no kernels, headers, tables, constant generators, pre- or
post-processing); the only module both sides use is the seeded input
generator ``synth``, which holds none of the method's arithmetic.

Sources (cited by page title and section):

* [QLoRA-074] "074｜QLoRA：把大模型放进显存，再用小适配器改变它"
  (wq-win.github.io/llm/074-qlora.html), a summary of Dettmers, Pagnoni,
  Holtzman, Zettlemoyer, "QLoRA: Efficient Finetuning of Quantized LLMs"
  (2023).  Sections used: §一 problem setting (the layer equation and what
  "frozen" means), §二 NF4 / double quantization, the boxed note on counting
  quantization constants in the compression ratio (including the
  self-constructed 16384-weight example), the note on what the backward pass
  still needs, §三 (the training procedure and the 4096×4096 example), §四
  Table 2 (the 4-bit format comparison) and §五/§六 on merging an adapter and
  quantizing again.
* [QLoRA-glossary] weimeta.cn glossary entry "QLoRA", section "NF4 4-bit
  量化是什么" (NF4 cuts the normal curve into 16 quantile intervals), and
  its FAQ on deployment (one 4-bit base, unmerged adapters per customer).
* [LoRA-PyTorch] "深入理解 LoRA 与 QLoRA低秩自适应微调的矩阵分解原理与
  PyTorch 高效实现" (mhpn.cn), §四.5 on switching between several adapters.

Arithmetic is fp64 (or exact) except where the method fixes fp32 / bf16
storage: the codebook and the scales are fp32 values, the dequantized weight
is an fp32 product rounded to bf16.

Modules:
  nf4     -- codebook, blockwise NF4 encode, double quantization, dequant.
  linear  -- forward / backward of Y = X·Ŵ + s·X·A·B in fp64.
  formats -- the int4 / FP4 comparison tables through the same scheme.
  dq      -- second-level variants centred on the tensor mean (int8, FP8).
  multi   -- one base with a LoRA adapter chosen per token.
  merge   -- the adapter merged into the base, then quantized again.
  adamw   -- the (paged) optimizer step of the adapter parameters.
"""

from . import nf4, linear, formats, dq, multi, merge, adamw  # noqa: F401
