"""CPU oracle for the fp9 routed-expert MoE FFN.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  The
product library (``bit_moe_expert_fp9_amd``) never imports it, and this package
imports nothing from the product: the two share no code, no tables and no
constants.

Everything here is plain numpy in float64 (the pages fix no precision for the
reference computation, so the oracle takes the widest one).  It is slow on
purpose: no blocking, no fusion, no reordering beyond the definitions.

Sources, cited by page title and section:

* duck-llm memoir page, "一鸭三吃：我把评测鸭变成了满血 DeepSeek-V3.2 推理系统":
  - section "在只有 AVX2 的 N100 上，我先做出了单核 MLP fp9" (the fp9 section:
    bit-layout figure, split body/sign storage, fp16-aligned decode);
  - section "真正埋下伏笔的是内存；R1 之后，问题第一次被改写" (FFN/MoE expert
    weights are what is spread over the boxes);
  - section "真正难的不是把参数塞下，而是通信" (tensor parallelism chosen);
  - section "先用 Qwen3 练级，再让 Qwen3.5 充当高压试炼场" (sub-128 TP slices,
    multiple_of 64/32);
  - section "16 tok/s 之后：一段没有跑通的路" (MoE forward breakdown block:
    per-box partials, host reduce);
  - the memory section above and the Qwen3 section (fp8 checkpoints with a
    128 x 128 block-scale format; converted to fp9 by ``fp8.py``).
* chapter page "第 9 章 MTP1 dual-lane overlap", section 9.2 "两条路线的判断"
  (route one: bsz=2, top_k=8 routed experts per token, near-disjoint sets);
  section 9.5 (the GPU stage normalises between layers: the stack glue).
* memoir page, section "限制条件" (the fp9 prefill kernel is the open item;
  contexts up to 2048 tokens): the per-expert token lists of ``prefill_plan``.
* ds4 glossary page "张量并行（Tensor Parallelism, TP）", section
  "形态一：Mac-to-Mac 张量并行（RDMA）" (TP partial sums are f32).

Parity status: every public function is pinned by ``tests/test_oracle_*.py``
against closed forms, an independent library route (numpy float16), brute
force, or exact rational arithmetic.  Unpinned: the payload bits of the 14 NaN
codes (only their NaN class is pinned).
"""

from .fp9 import (  # noqa: F401
    FP9_MAX,
    decode,
    quantize,
    quantize_f64,
    pack,
    unpack,
    decode_planes,
)
from .fp8 import (  # noqa: F401
    E4M3_MAX,
    decode_e4m3,
    dequantize,
    fp8_to_fp9,
)
from .moe import (  # noqa: F401
    gemv,
    silu,
    expert_ffn,
    moe_plan,
    moe_slot_weights,
    moe_layer,
    moe_partials,
    prefill_plan,
    rms_normalize,
)
