"""Model shapes and draft/base pair configurations.

The five pair configurations are the synthetic workloads the method is measured
on: Llama- and Qwen-shaped decoder pairs with random-init weights.  The pages
of "EasySpec: Layer-Parallel Speculative Decoding for Efficient Multi-GPU
Utilization" evaluate same-family drafter/base pairs (LLaMA-3 and Qwen2
families, rebuttal replies on Table 8 and on the smaller-drafter question) with
draft length 5 and generation lengths of at most 128 tokens (reply on the
optimal TP size); these shapes stand in for those checkpoints.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field
from typing import Tuple

F32 = 0
BF16 = 1


@dataclass(frozen=True)
class ModelShape:
    n_layers: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    d_ffn: int
    vocab: int
    qkv_bias: bool = False
    dtype: int = BF16          # F32 or BF16 (weights and KV cache)
    rms_eps: float = 1e-5
    rope_theta: float = 500000.0

    @property
    def qkv_rows(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim

    @property
    def q_dim(self) -> int:
        return self.n_q_heads * self.head_dim

    def n_params(self) -> int:
        d, L = self.d_model, self.n_layers
        per_layer = self.qkv_rows * d + d * self.q_dim + 3 * self.d_ffn * d
        return L * per_layer + 2 * self.vocab * d

    def replace(self, **kw) -> "ModelShape":
        return dataclasses.replace(self, **kw)


@dataclass(frozen=True)
class PairConfig:
    name: str
    index: int
    draft: ModelShape
    base: ModelShape
    prompt_len: int
    k: int                      # draft tokens per round
    group_size: int             # layer-parallel set size N
    new_tokens: int
    batch: int
    temperatures: Tuple[float, ...] = (0.0,)

    @property
    def seed_draft(self) -> int:
        return 1000 * self.index + 1

    @property
    def seed_base(self) -> int:
        return 1000 * self.index + 2

    def prompt_seed(self, b: int) -> int:
        return 2000 * self.index + b

    @property
    def sample_seed(self) -> int:
        return 3000 * self.index

    @property
    def capacity(self) -> int:
        # every position a round may touch: prompt + new tokens + one full round
        return self.prompt_len + self.new_tokens + self.k + 2


def tiny_shape(n_layers=2, d_model=64, n_q_heads=4, n_kv_heads=4, head_dim=16,
               d_ffn=256, vocab=256, **kw) -> ModelShape:
    kw.setdefault("dtype", F32)
    kw.setdefault("rope_theta", 10000.0)
    return ModelShape(n_layers, d_model, n_q_heads, n_kv_heads, head_dim, d_ffn, vocab, **kw)


_LLAMA_1B = ModelShape(16, 2048, 32, 8, 64, 8192, 128256, False, BF16, 1e-5, 500000.0)
_LLAMA_8B = ModelShape(32, 4096, 32, 8, 128, 14336, 128256, False, BF16, 1e-5, 500000.0)
_LLAMA_70B = ModelShape(80, 8192, 64, 8, 128, 28672, 128256, False, BF16, 1e-5, 500000.0)
_QWEN_05B = ModelShape(24, 896, 14, 2, 64, 4864, 152064, True, BF16, 1e-6, 1000000.0)
_QWEN_7B = ModelShape(28, 3584, 28, 4, 128, 18944, 152064, True, BF16, 1e-6, 1000000.0)

CONFIGS = {
    "tiny": PairConfig("tiny-fp32", 0,
                       tiny_shape(2, 64, 4, 4, 16, 256, 256),
                       tiny_shape(4, 128, 4, 4, 32, 512, 256),
                       prompt_len=32, k=4, group_size=2, new_tokens=64, batch=1,
                       temperatures=(0.0, 1.0)),
    "llama-1b-8b": PairConfig("llama-1b-8b", 1, _LLAMA_1B, _LLAMA_8B,
                              prompt_len=512, k=5, group_size=2, new_tokens=128, batch=1,
                              temperatures=(0.0, 1.0)),
    "llama-1b-8b-n4": PairConfig("llama-1b-8b-n4", 2, _LLAMA_1B, _LLAMA_8B,
                                 prompt_len=2048, k=8, group_size=4, new_tokens=128, batch=1,
                                 temperatures=(0.0, 1.0)),
    "qwen-0.5b-7b": PairConfig("qwen-0.5b-7b", 3, _QWEN_05B, _QWEN_7B,
                               prompt_len=1024, k=6, group_size=3, new_tokens=128, batch=1,
                               temperatures=(0.7,)),
    "llama-8b-70b": PairConfig("llama-8b-70b", 4, _LLAMA_8B, _LLAMA_70B,
                               prompt_len=8192, k=6, group_size=4, new_tokens=128, batch=4,
                               temperatures=(0.0, 1.0)),
}
CONFIG_ORDER = ["tiny", "llama-1b-8b", "llama-1b-8b-n4", "qwen-0.5b-7b", "llama-8b-70b"]


def get_config(name_or_index) -> PairConfig:
    if isinstance(name_or_index, int):
        return CONFIGS[CONFIG_ORDER[name_or_index]]
    return CONFIGS[name_or_index]
