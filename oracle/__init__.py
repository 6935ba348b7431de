"""CPU oracle for the grouped NF4 MoE expert path -- TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, obviously-correct NumPy reference of what the
hot path computes.  It exists to check the HIP implementation and nothing
else: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import it.  The product library never imports,
links or calls anything in here, and this package imports nothing from the
product (it shares no code, tables or constants with it).

Sources (the pages are the text of the experts4bit-qlora / grouped-nf4-gemm
project pages):

* experts4bit-qlora 0.22.0 README, "The problem" and "Quickstart": the fused
  expert stacks ``gate_up_proj [E, 2I, H]`` and ``down_proj [E, H, I]``.
* "Why does load_in_4bit still OOM on a Mixture-of-Experts model?", section
  "Which project solves it": 4-bit blocks never cross an expert boundary.
* experts4bit-qlora 0.22.0 README, "Which door?" (enable_fast paragraph): NF4
  at blocksize 64, decoded inside the GEMM with fp32 accumulation.
* experts4bit-qlora 0.22.0 README, "Inference": the same codebook and the same
  per-expert absmax at train and serve time.
* Solutions index, "How do I QLoRA-train the fused experts": the per-expert
  LoRA delta is added before each routed expert's activation.
* experts4bit-qlora 0.22.0 README, "Which training path?": token/expert pairs
  are sorted and the experts are summed in group-sorted order.

Where the pages leave a step open (the 16 codebook values, the nibble order,
tie rules, the router formula) the reading taken is stated in the function
that implements it.

Parity status of every function is recorded in its module docstring; every
function here is pinned by ``tests/test_oracle_*.py`` against values the pages
print, closed forms, brute force or library routines.
"""

from .nf4 import (  # noqa: F401
    BLOCKSIZE,
    nf4_codebook,
    nf4_codebook_f64,
    nf4_levels_unnormalised,
    fp4_codebook,
    fp4_codebook_f64,
    fp4_code,
    codebook,
    QUANT_TYPES,
    block_error_bound,
    nearest_code,
    quantize_blockwise,
    dequantize_blockwise,
    unpack_codes,
    pack_codes,
    packed_bytes,
)
from .routing import route_topk, permute_pairs  # noqa: F401
from .moe import (  # noqa: F401
    silu,
    expert_mlp,
    grouped_gemm,
    moe_forward,
    moe_forward_tokens,
)
from .backward import (  # noqa: F401
    silu_grad,
    swiglu_backward,
    grouped_dgrad,
    expert_backward,
    moe_backward,
    moe_backward_tokens,
)
from .mxfp4 import (  # noqa: F401
    MX_BLOCK,
    e2m1_value,
    e8m0_value,
    unpack_mx,
    pack_mx,
    dequantize_mxfp4,
    grouped_gemm_mxfp4,
    moe_forward_mxfp4,
)
from .passthrough import (  # noqa: F401
    PASSTHROUGH,
    bf16_store,
    bf16_value,
    fp16_store,
    fp16_value,
    store16,
    value16,
    grouped_gemm16,
    moe_forward16,
)
from .nbit8 import (  # noqa: F401
    e4m3_value,
    int8_code,
    fp8_code,
    quantize_blockwise8,
    dequantize_blockwise8,
)
