"""CPU oracle for the paged-attention path -- TEST INFRASTRUCTURE ONLY.

A plain, slow, fp64 NumPy statement of what the path computes: the
reshape-and-cache scatter and causal softmax attention of packed query rows
over a KV cache held in 16-token physical blocks.  It shares no code with the
HIP path and must never be imported by the product package; only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline leg use it.

Sources (web pages, cited by title and section):
  * "【大模型基础设施工程】12：PagedAttention 与 Continuous Batching" (quant67),
    §3.2 (KV cut into fixed blocks, block table), §3.3 (data structures and
    the worked address example; per-decode-step order: write new K/V, then
    attend), §3.6 (the kernel walks block_table and accumulates an online
    softmax; the result equals ordinary attention), §3.7 (16 tokens per block),
    §4 (chunked prefill), §10.8 FAQ (shared-prefix reuse is mathematically
    identical up to rounding).
    §3.8 (reference counts and copy-on-write), §3.9 (swap), §5.2 (prefix
    keys and LRU eviction) for the block manager and block copies.
  * "推理优化与服务：从 PagedAttention 到分离式部署" (ice-wocker), latest
    developments: query tokens packed as [total_q, H, D] with cu_seqlens
    request boundaries in one mixed prefill/decode step.

Parity pins: every function here is pinned by CPU tests against worked
examples from the pages, closed forms, invariances and an independently
written brute force.  What no pin reaches is said so in the function.
"""

from .paged_attention import (  # noqa: F401
    OracleError,
    compare_outputs,
    fp8_e4m3_decode,
    fp8_e4m3_encode,
    fp8_quantize_rows,
    first_visible_key,
    gather_request_kv,
    kv_head_of,
    last_visible_key,
    oracle_attention_varlen,
    oracle_cache_write,
    physical_location,
    validate_metadata,
    widen,
)
from .block_manager import (  # noqa: F401
    OracleBlockManager,
    OutOfBlocks,
    oracle_copy_blocks,
    oracle_swap_blocks,
)
