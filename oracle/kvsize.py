"""KV-cache size and waste arithmetic from the pages.  TEST INFRASTRUCTURE ONLY.

Per-token bytes ([Serving] "What the KV Cache Is, and How Big It Gets"): two vectors (K and V)
per layer per KV head, each head_dim values of p bytes:
    bytes/token = 2 * layers * kv_heads * head_dim * p.
Whole cache ([Walkthrough] "Step 5" and "Feynman retelling"): 2 * B * S * L * d_model * p, where
d_model = n_head * d_head ("Step 3").  The two agree when every query head has its own KV head;
with grouped-query attention the KV-head form is the right one ([Serving] scales its figures by
the KV-head count: quadrupling the KV heads quadruples every size).

Waste ([Walkthrough] "Step 6", "Step 7", "Step 8", "Quick self-check"): a contiguous
reservation of max_len tokens wastes max_len - S slots; paging wastes only the empty tail of the
last block, ceil(S / bs) * bs - S, which is at most bs - 1.
"""
from __future__ import annotations


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, bytes_per_value: float):
    return 2 * layers * kv_heads * head_dim * bytes_per_value


def kv_bytes_total(batch: int, seq_len: int, layers: int, d_model: int, bytes_per_value: float):
    return 2 * batch * seq_len * layers * d_model * bytes_per_value


def blocks_for(tokens: int, block_size: int) -> int:
    return -(-tokens // block_size)


def paged_waste(tokens: int, block_size: int) -> int:
    return blocks_for(tokens, block_size) * block_size - tokens


def naive_waste(tokens: int, max_len: int) -> int:
    return max_len - tokens
