"""CPU float64 oracle for exact, tiled and paged attention.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
execute this package: it is used by ``tests/``, by ``__graft_entry__.smoke()``
and by the ``cpu_baseline`` leg of ``bench.py``, and by nothing else. It shares
no code with the HIP library or its Python binding; the only module both sides
use is ``workloads`` (seeded input generators, which hold none of the method's
arithmetic).

Sources (the web pages this library follows; sections as they appear there):
  [P1] iopencloud.com, "大模型推理加速技术全景：从FlashAttention到Speculative
       Decoding" -- §2.1 (standard attention), §2.2 (tiling + online softmax
       pseudocode), §3.2 (paging, KV block pool figure).
  [P2] ybb.press/llm-inference/15723.html -- §一 (scaled dot-product attention
       formula), §三 (Flash Attention, A100 comparison table).
  [P3] lowentro.cn notes, "推理加速技术" -- Q&A items on the FlashAttention core
       idea, FlashAttention-2, FlashDecoding, and Continuous Batching with
       PagedAttention (block tables passed to the kernel).
  [P4] fanzheng.org, "a survey of advances in LLM since the transformer:
       inference" -- roofline, MFU/MBU, PagedAttention (16-token blocks,
       reference-counted physical blocks copied on write).

Every function here is pinned by tests that do not re-run its own formula
(brute-force scalar loops, a library routine, closed forms, invariants and a
hand-checkable fixture from [P1] §3.2); no function is "parity unpinned".
"""

from .attention import (  # noqa: F401
    causal_visibility,
    masked_attention,
    dense_attention,
    prefill,
    block_state,
    combine_states,
    online_softmax_attention,
    paged_gather,
    paged_attention,
    paged_attention_varlen,
    split_ranges,
    split_partials,
    lse_merge,
)
from .cache import paged_append, copy_blocks  # noqa: F401,E402
from .fp8 import (  # noqa: F401,E402
    E4M3_MAX,
    e4m3_decode,
    e4m3_encode,
    quantize_append,
    dequantize,
    paged_attention_fp8,
)
