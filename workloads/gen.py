"""Seeded draws: Q/K/V tensors, document cuts, decode cache lengths, row samples.

Rules (the same for every caller, so oracle and kernels see identical inputs):

* tensors: ``torch.Generator('cpu').manual_seed(seed)``; standard-normal fp32
  draws taken in the order Q, K, V (decode: Q, then K and V of each sequence in
  batch order), then cast to the storage dtype (bf16 rounds to nearest even);
* documents: ``numpy.random.default_rng(seed + 1)``; the document count is
  drawn from U{1..n_docs_max} unless fixed, and the n_docs - 1 interior cuts are
  drawn without replacement from {1, ..., S-1}, so every document is non-empty;
* decode lengths: ``numpy.random.default_rng(seed + 1)``, L_b ~ U{lo..hi}
  inclusive, where L_b counts the new token;
* sampled rows: ``numpy.random.default_rng(seed + 2)``.
"""

from __future__ import annotations

from typing import List, Optional, Tuple

import numpy as np
import torch

_TORCH_DTYPE = {"fp32": torch.float32, "bf16": torch.bfloat16}


def torch_dtype(name: str) -> torch.dtype:
    return _TORCH_DTYPE[name]


def _randn(shape, gen: torch.Generator, dtype: str) -> torch.Tensor:
    return torch.randn(*shape, generator=gen, dtype=torch.float32).to(_TORCH_DTYPE[dtype])


def draw_cu_docs(S: int, seed: int, n_docs: Optional[int] = None,
                 n_docs_max: int = 1) -> np.ndarray:
    """Document offsets [n_docs + 1] int32: 0 = b_0 < b_1 < ... < b_n = S."""
    if S < 1:
        raise ValueError("S must be >= 1")
    rng = np.random.default_rng(seed + 1)
    if n_docs is None:
        n_docs = int(rng.integers(1, n_docs_max + 1))
    n_docs = min(n_docs, S)
    cuts = np.sort(rng.choice(np.arange(1, S), size=n_docs - 1, replace=False)) if n_docs > 1 \
        else np.zeros(0, dtype=np.int64)
    return np.concatenate([[0], cuts, [S]]).astype(np.int32)


def draw_seq_lens(B: int, lo: int, hi: int, seed: int) -> np.ndarray:
    """Decode cache lengths [B] int32, each uniform in {lo..hi} inclusive."""
    rng = np.random.default_rng(seed + 1)
    return rng.integers(lo, hi + 1, size=B).astype(np.int32)


def draw_prefill_inputs(B: int, S: int, Hq: int, Hkv: int, D: int, dtype: str,
                        seed: int) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Q [B,S,Hq,D], K [B,S,Hkv,D], V [B,S,Hkv,D] on the CPU, N(0,1) draws."""
    gen = torch.Generator("cpu").manual_seed(seed)
    q = _randn((B, S, Hq, D), gen, dtype)
    k = _randn((B, S, Hkv, D), gen, dtype)
    v = _randn((B, S, Hkv, D), gen, dtype)
    return q, k, v


def draw_grad_output(B: int, S: int, Hq: int, D: int, dtype: str, seed: int) -> torch.Tensor:
    """The output gradient dL/dO of a backward pass: standard normal [B, S, Hq, D]
    (its own stream: seed + 7919)."""
    gen = torch.Generator("cpu").manual_seed(seed + 7919)
    return _randn((B, S, Hq, D), gen, dtype)


def draw_decode_inputs(B: int, Hq: int, Hkv: int, D: int, seq_lens, dtype: str,
                       seed: int) -> Tuple[torch.Tensor, List[torch.Tensor], List[torch.Tensor]]:
    """Decode inputs on the CPU.

    Returns the new tokens' raw query q [B,Hq,D] and, per sequence b, the raw
    (unrotated) keys and the values of its L_b cached tokens as [Hkv, L_b, D];
    slot L_b - 1 holds the new token's own key and value.
    """
    gen = torch.Generator("cpu").manual_seed(seed)
    q = _randn((B, Hq, D), gen, dtype)
    ks, vs = [], []
    for b in range(B):
        L = int(seq_lens[b])
        ks.append(_randn((Hkv, L, D), gen, dtype))
        vs.append(_randn((Hkv, L, D), gen, dtype))
    return q, ks, vs


def draw_positions(B: int, S: int, max_pos: int, seed: int) -> np.ndarray:
    """Arbitrary token positions [B,S] int32 in [0, max_pos]."""
    rng = np.random.default_rng(seed + 3)
    return rng.integers(0, max_pos + 1, size=(B, S)).astype(np.int32)


def sample_rows(S: int, cu_docs, seed: int, n_random: int = 2048,
                tile: int = 64, n_edges: Optional[int] = None) -> np.ndarray:
    """Query rows to check at sizes where the oracle cannot do every row.

    Every document's first and last row, rows either side of tile edges
    (multiples of ``tile``; at most ``n_edges`` of them, drawn, when given) and
    ``n_random`` uniformly drawn rows; sorted and unique.
    """
    rng = np.random.default_rng(seed + 2)
    cu = np.asarray(cu_docs, dtype=np.int64)
    rows = [cu[:-1], cu[1:] - 1]
    edges = np.arange(tile, S, tile, dtype=np.int64)
    if n_edges is not None and edges.size > n_edges:
        edges = rng.choice(edges, size=n_edges, replace=False)
    rows += [edges - 1, edges]
    if n_random > 0:
        rows.append(rng.integers(0, S, size=n_random))
    r = np.unique(np.concatenate(rows))
    return r[(r >= 0) & (r < S)]
