"""KV-cache sizing closed form and block-count arithmetic (O4).

KV bytes = 2 (K and V) x layers x kv_heads x head_dim x seq_len x batch x
bytes per element ([P2] question 1, sub-section 1.2 compute_kv_cache_memory;
with GQA/MQA the kv head count replaces the query head count, 1.1; fp8 uses
one byte, 1.3; tensor parallelism divides by the number of ways, 1.4; the
same form in [P3] code block kv_cache_memory).

Blocks needed for L tokens = ceil(L / block_size); logical block i covers
tokens [i*bs, min((i+1)*bs, L)) ([P2] question 14,
build_block_table_for_prefill; [P1] `BlockTableDesign.table_structure`).

Pins (tests/test_oracle_sizing.py): the pages' printed figures, stored with
their citations in tests/golden/.
"""

from __future__ import annotations

from typing import List, Tuple


def kv_cache_bytes(num_layers: int, num_kv_heads: int, head_dim: int,
                   seq_len: int, batch: int, dtype_bytes: float = 2,
                   tp_ways: int = 1) -> float:
    per_token_layer = 2 * num_kv_heads * head_dim * dtype_bytes
    return num_layers * batch * seq_len * per_token_layer / tp_ways


def blocks_needed(num_tokens: int, block_size: int) -> int:
    return -(-num_tokens // block_size)


def block_ranges(num_tokens: int, block_size: int) -> List[Tuple[int, int]]:
    return [(i * block_size, min((i + 1) * block_size, num_tokens))
            for i in range(blocks_needed(num_tokens, block_size))]


def tokens_in_last_block(num_tokens: int, block_size: int) -> int:
    if num_tokens == 0:
        return 0
    r = num_tokens % block_size
    return block_size if r == 0 else r
