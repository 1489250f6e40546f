"""Plain, slow, CPU-only oracle for the QLoRA NF4 + double-quantization + LoRA linear.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or link
this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, table or
constant generator with the HIP library in ``bit_quantized_lora_nf4_amd``.

Pages cited (titles and sections as printed on each page):

* [QLoRA note]  "1. 啥是 QLoRA" (p19e99.github.io/posts/note/qlora),
  sections "2. NF4", "3. 双重量化", "5. QLoRA 训练方式本身".
* [Ch. 11.3]    "11.3 QLoRA：单卡微调大模型" (gheillcoat.github.io),
  sections "核心创新一：NF4 数据类型", "核心创新二：双重量化".
* [Paper note]  "QLoRA — 让 65B 大模型微调落到单张 48GB GPU 上"
  (awesome.papernotes.org), sections "关键设计 1/2/3" and the
  ``qlora_linear`` listing under "关键设计 3".
* [Digest]      "QLoRA: 高效微调量化大语言模型" (aipaper.cc), section
  "4. 方法论": "方法步骤与流程" and "数学公式与关键细节" items 1-3.
* [Repro]       "LoRA / QLoRA低秩更新、量化和显存预算" (mhpn.cn), sections
  "LoRA 的公式和张量形状" and "最小实验与验收协议".

Module map:

* ``oracle.fp``         exact IEEE helpers (bf16 RNE, single-rounding fma).
* ``oracle.nf4``        codebook, thresholds, blockwise NF4 quantization,
                        double quantization, decoding.
* ``oracle.linear``     forward / backward of the linear layer in float64.
* ``oracle.accounting`` closed-form storage and parameter counts.
* ``oracle.adamw``      the AdamW step on the adapter parameters.
* ``oracle.merge``      LoRA merge / unmerge into a bf16 copy of the base.
* ``oracle.fusion``     horizontally fused linears (stacked weights and adapters).
* ``oracle.variants``   FP4 levels, FP8-coded and fp32 block constants.

Every function is pinned by ``tests/test_oracle_*.py`` to facts the pages or
mathematics fix; none is "parity unpinned".
"""

from . import fp, nf4, linear, accounting, adamw, merge, fusion, variants  # noqa: F401

__all__ = ["fp", "nf4", "linear", "accounting", "adamw", "merge", "fusion", "variants"]
