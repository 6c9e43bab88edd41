"""The five workloads the library is checked and measured on.

Shapes follow the pages' training setting (Qwen3-4B/8B-shaped attention:
32 query heads, 8 KV heads, head_dim 128; 128 groups x 8 responses, 16,384
token response cap; run-wide mean response length about 1.45k -- news
summary "Async RL squeezes context into fewer decode steps ...",
Interpretation paragraphs 3 and 4).  Distribution parameters the pages leave
open (lognormal sigma, outlier channels) are readings, listed per field.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Tuple


@dataclass(frozen=True)
class Config:
    idx: int
    name: str
    seed: int
    layers: int
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    n_sink: int
    n_recent: int
    n_outlier: int
    # context lengths: exactly one of these is used
    fixed_lengths: Optional[Tuple[int, ...]] = None
    prompt_len: int = 0            # tokens before the response
    resp_mean: float = 0.0         # lognormal response mean (tokens)
    resp_sigma: float = 1.0        # lognormal sigma (reading)
    resp_cap: int = 16384          # response cap
    uniform: Optional[Tuple[int, int]] = None  # uniform context range
    group: int = 1                 # sequences sharing one prompt
    page_size: int = 16
    group_size: int = 32
    note: str = field(default="", compare=False)

    @property
    def g(self) -> int:
        return self.num_q_heads // self.num_kv_heads


CONFIGS = {
    0: Config(0, "tiny-d64", 1000, 1, 2, 4, 2, 64, 4, 16, 4, fixed_lengths=(300, 517),
              note="CPU-seconds case: contexts 300 and 517"),
    1: Config(1, "qwen3-4b-layer-b128", 1001, 1, 128, 32, 8, 128, 16, 128, 6,
              prompt_len=256, resp_mean=1450.0,
              note="256-token prompt + lognormal response (mean 1.45k, cap 16,384)"),
    2: Config(2, "qwen3-8b-layer-b1024", 1002, 1, 1024, 32, 8, 128, 16, 128, 6,
              prompt_len=256, resp_mean=2000.0, group=8,
              note="128 groups x 8 responses, shared 256-token prompt, "
                   "lognormal response (mean 2k, cap 16,384)"),
    3: Config(3, "qwen3-8b-36-layers-b512", 1003, 36, 512, 32, 8, 128, 16, 128, 6,
              uniform=(4096, 16600),
              note="36 layers, contexts uniform in [4096, 16600]"),
    4: Config(4, "precision-ablation-b1024", 1002, 1, 1024, 32, 8, 128, 16, 128, 6,
              prompt_len=256, resp_mean=2000.0, group=8,
              note="config-2 shapes and data; BF16 / INT8 / plain INT4 / KV4-RL"),
}


def get_config(idx: int) -> Config:
    return CONFIGS[int(idx)]
