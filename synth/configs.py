"""The paged-decode workloads, by shape.

Shapes follow the paged layout [num_blocks, block_size, num_kv_heads,
head_dim] used by the `paged_attention` code block of the page
"paged-attention-and-vllm-inference" (astro-blog-cod.pages.dev).  The model
shapes are the LLaMA-2 7B / 70B attention shapes the pages size their KV
caches with (page "5.KV Cache 管理 & PagedAttention", question 1; same page,
question 7 for the 64 q-head / 8 kv-head grouping of 70B).
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Tuple


@dataclass(frozen=True)
class WorkloadConfig:
    name: str
    description: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    q_dtype: str  # "f32" | "f16" | "bf16"
    kv_dtype: str  # "f32" | "f16" | "bf16" | "fp8"
    # length recipe: ("fixed", L) | ("uniform", lo, hi) | ("lognormal", mu, sigma, lo, hi)
    lengths: Tuple
    # physical pool = ceil(pool_factor * blocks needed) (+ shared prefix blocks)
    pool_factor: float = 1.25
    # explicit pool size (overrides pool_factor when > 0)
    pool_blocks: int = 0
    # leading tokens of every sequence that live in ref-counted shared blocks
    shared_prefix_tokens: int = 0
    seed: int = 0
    tags: Tuple[str, ...] = field(default_factory=tuple)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def src_dtype(self) -> str:
        """dtype of the K/V tokens handed to the cache write."""
        return self.q_dtype if self.kv_dtype == "fp8" else self.kv_dtype


CONFIGS: Dict[str, WorkloadConfig] = {}


def _add(c: WorkloadConfig) -> None:
    CONFIGS[c.name] = c


_add(WorkloadConfig(
    name="tiny_mha_fp32",
    description="1 sequence of 100 tokens (last block 4/16), 4 heads, d=64, "
                "bs=16, 64-block pool, fp32",
    batch=1, num_q_heads=4, num_kv_heads=4, head_dim=64, block_size=16,
    q_dtype="f32", kv_dtype="f32", lengths=("fixed", 100), pool_blocks=64,
    seed=1001))

_add(WorkloadConfig(
    name="llama2_7b_decode_fp16",
    description="batch 32, 32 q = 32 kv heads, d=128, bs=16, "
                "seq_lens uniform in [512, 2048], fp16, pool 1.25x need",
    batch=32, num_q_heads=32, num_kv_heads=32, head_dim=128, block_size=16,
    q_dtype="f16", kv_dtype="f16", lengths=("uniform", 512, 2048),
    seed=1002))

_add(WorkloadConfig(
    name="llama2_70b_gqa_decode_bf16",
    description="batch 64, 64 q / 8 kv heads (group 8), d=128, bs=16, "
                "seq_len 4096, bf16",
    batch=64, num_q_heads=64, num_kv_heads=8, head_dim=128, block_size=16,
    q_dtype="bf16", kv_dtype="bf16", lengths=("fixed", 4096), seed=1003))

_add(WorkloadConfig(
    name="long_context_split_bf16",
    description="batch 4, seq_len 32768, 32 q / 8 kv heads, d=128, bs=16, "
                "bf16, 512-token partitions merged by the reduce kernel",
    batch=4, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
    q_dtype="bf16", kv_dtype="bf16", lengths=("fixed", 32768), seed=1004,
    tags=("split",)))

_add(WorkloadConfig(
    name="mixed_shared_prefix_fp8",
    description="batch 128, seq_lens lognormal(7, 1) clipped to [16, 16384], "
                "first 1024 tokens in shared ref-counted prefix blocks, "
                "32 q / 8 kv heads, d=128, bs=32, K/V fp8 e4m3 (per-tensor "
                "scale), Q bf16",
    batch=128, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=32,
    q_dtype="bf16", kv_dtype="fp8", lengths=("lognormal", 7.0, 1.0, 16, 16384),
    shared_prefix_tokens=1024, seed=1005))

_add(WorkloadConfig(
    name="shared_system_prompt_decode_bf16",
    description="200 requests sharing a 512-token system prompt (32 ref-counted "
                "blocks of 16), each with 16..256 tokens of its own after it "
                "(seq_lens uniform in [528, 768]), 64 q / 8 kv heads, d=128, "
                "bs=16, bf16",
    batch=200, num_q_heads=64, num_kv_heads=8, head_dim=128, block_size=16,
    q_dtype="bf16", kv_dtype="bf16", lengths=("uniform", 528, 768),
    shared_prefix_tokens=512, seed=1006))

# Ordered as listed above; index 0 is the small case, index 1 the bench case.
CONFIG_ORDER = list(CONFIGS)

# Prefill workloads: the cache holds each sequence's tokens (drawn as for
# decode); a prefill call brings the last `new_tokens` of them as query rows
# (synth.generate.make_prefill_rows).  Same model shapes as above.
PREFILL_CONFIGS: Dict[str, Tuple[WorkloadConfig, Tuple]] = {}


def _add_prefill(c: WorkloadConfig, new_tokens: Tuple) -> None:
    PREFILL_CONFIGS[c.name] = (c, new_tokens)


_add_prefill(WorkloadConfig(
    name="llama2_7b_prefill_fp16",
    description="8 prompts of 2048 tokens, whole-prompt causal prefill, "
                "32 q = 32 kv heads, d=128, bs=16, fp16",
    batch=8, num_q_heads=32, num_kv_heads=32, head_dim=128, block_size=16,
    q_dtype="f16", kv_dtype="f16", lengths=("fixed", 2048), seed=2001), ("all",))

_add_prefill(WorkloadConfig(
    name="llama2_70b_gqa_chunked_prefill_bf16",
    description="4 sequences of 4096 tokens, the last 1024 as one prefill "
                "chunk over 3072 cached tokens, 64 q / 8 kv heads, d=128, "
                "bs=16, bf16",
    batch=4, num_q_heads=64, num_kv_heads=8, head_dim=128, block_size=16,
    q_dtype="bf16", kv_dtype="bf16", lengths=("fixed", 4096), seed=2002),
    ("fixed", 1024))


def get_prefill_config(name: str) -> Tuple[WorkloadConfig, Tuple]:
    aliases = {f"p{i + 1}": n for i, n in enumerate(PREFILL_CONFIGS)}
    return PREFILL_CONFIGS[aliases.get(name, name)]


def get_config(name_or_index) -> WorkloadConfig:
    if isinstance(name_or_index, int):
        return CONFIGS[CONFIG_ORDER[name_or_index]]
    if name_or_index in CONFIGS:
        return CONFIGS[name_or_index]
    aliases = {f"c{i + 1}": n for i, n in enumerate(CONFIG_ORDER)}
    return CONFIGS[aliases[name_or_index]]
