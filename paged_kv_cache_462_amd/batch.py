"""Building a decode batch through the host block manager and prefix cache.

Host code only: every step is a call into libpa.so (the allocator, the
sequence block manager, the prefix cache); nothing here touches the device.

The case covered is a batch of requests that start with one shared prompt
(a system prompt shared by many requests: "KV Cache 优化与内存管理深度解析：
PagedAttention 原理与实践", `HashBasedCaching`; "5.KV Cache 管理 &
PagedAttention", question 20, allocate_with_prefix;
"paged-attention-and-vllm-inference", `PrefixCacheManager`).  The prompt is
admitted first, as a sequence of its own, and its full blocks enter the
prefix cache; then each request is admitted through the cache, so its table
starts with the prompt's blocks (one reference each) and blocks are
allocated for the rest; finally the prompt's own sequence is released, and
its blocks live on through the cache's reference and the requests'.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import List, Sequence, Tuple

import numpy as np

from .ops import BlockManager, PrefixCache


@dataclass
class AdmittedBatch:
    seq_ids: List[int]
    tables: np.ndarray          # [B, max_blocks] int32, -1 padded
    seq_lens: np.ndarray        # [B] int32
    matched: np.ndarray         # [B] tokens each request found in the cache
    prompt_blocks: np.ndarray   # physical blocks holding the prompt
    # K/V the caller must write before decoding: (request index, or -1 for
    # the prompt; first position; slots of positions first, first + 1, ...)
    writes: List[Tuple[int, int, np.ndarray]]


def admit_with_shared_prompt(manager: BlockManager, cache: PrefixCache,
                             prompt_ids: Sequence[int], requests: Sequence[Sequence[int]],
                             max_blocks: int, first_seq_id: int = 0,
                             prompt_seq_id: int = -1) -> AdmittedBatch:
    """Admit the shared prompt, then every request (token ids, the prompt's
    first), through pa_bm_add_sequence_cached; release the prompt's own
    sequence; export the requests' tables."""
    writes: List[Tuple[int, int, np.ndarray]] = []
    k, slots = manager.add_sequence_cached(cache, prompt_seq_id, prompt_ids)
    writes.append((-1, k, slots))
    nb = manager.num_blocks_of(prompt_seq_id)
    ptab, _ = manager.export([prompt_seq_id], max(nb, 1))
    prompt_blocks = ptab[0, :nb].copy()
    seq_ids, matched = [], []
    for i, toks in enumerate(requests):
        sid = first_seq_id + i
        k, slots = manager.add_sequence_cached(cache, sid, toks)
        writes.append((i, k, slots))
        seq_ids.append(sid)
        matched.append(k)
    manager.free_sequence(prompt_seq_id)
    tables, lens = manager.export(seq_ids, max_blocks)
    return AdmittedBatch(seq_ids=seq_ids, tables=tables, seq_lens=lens,
                         matched=np.asarray(matched, dtype=np.int64),
                         prompt_blocks=prompt_blocks, writes=writes)
