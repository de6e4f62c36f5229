"""The five workloads the attention path is checked and measured on.

Shapes follow the pages: the 405B layer has 128 query heads sharing 8 KV heads
(16:1) with head_dim 16384/128 = 128 ("Llama 3.1 Architecture: Dense Scaling to
405B and 128K Context", flowchart in "Architectural Deep Dive"); GQA with 8 KV
heads, RoPE base 500,000 and a cross-document mask ("The Llama 3 Herd of
Models", Chapter Roadmap, "A Deliberately Standard Dense Transformer"); a 128K
context window (same page, "Paper Overview"). The 8B layer's 32 query heads are
not printed on the pages; they are the workload's stated shape.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str                 # "prefill" or "decode"
    B: int
    S: int                    # prefill: tokens per sequence; decode: 1 new token
    Hq: int
    Hkv: int
    D: int
    dtype: str                # "fp32" or "bf16": the dtype Q/K/V are stored in
    seed: int
    n_docs: Optional[int] = None      # fixed document count (None: drawn)
    n_docs_max: int = 1               # upper end of the U{1..n_docs_max} draw
    len_lo: int = 0                   # decode: cache length range, inclusive
    len_hi: int = 0
    rope_base: float = 500000.0

    @property
    def group(self) -> int:
        return self.Hq // self.Hkv


CONFIGS = {
    "tiny": Workload("tiny", "prefill", B=1, S=128, Hq=8, Hkv=2, D=64,
                     dtype="fp32", seed=1, n_docs=1),
    "llama8b": Workload("llama8b", "prefill", B=1, S=8192, Hq=32, Hkv=8, D=128,
                        dtype="bf16", seed=2, n_docs_max=8),
    "llama405b": Workload("llama405b", "prefill", B=1, S=32768, Hq=128, Hkv=8,
                          D=128, dtype="bf16", seed=3, n_docs_max=8),
    "decode405b": Workload("decode405b", "decode", B=16, S=1, Hq=128, Hkv=8,
                           D=128, dtype="bf16", seed=4, len_lo=4096,
                           len_hi=131072),
    "long128k": Workload("long128k", "prefill", B=1, S=131072, Hq=128, Hkv=8,
                         D=128, dtype="bf16", seed=5, n_docs=4),
}


def get(name: str) -> Workload:
    return CONFIGS[name]
