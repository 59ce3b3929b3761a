"""Host-side arithmetic of the three methods (positions and budgets).

Small integer computations that decide the arguments of the library calls:
where each re-positioned unit starts and how many units are kept.
"""

from __future__ import annotations

from fractions import Fraction
from typing import Sequence

import torch


def reuse_window_starts(n_docs: int, doc_len: int, window: int) -> list:
    """Start position of each document cache under CacheFocus's adaptive
    re-positioning (§2.3.1): at most ``window // doc_len`` caches fit the
    positional range with unique positions; consecutive runs of that many
    documents form one group whose caches get sequential positions, and every
    group reuses the range from 0."""
    per_group = max(1, window // doc_len)
    return [doc_len * (i % per_group) for i in range(n_docs)]


def reuse_count(n_docs: int, doc_len: int, window: int) -> int:
    """N_reuse of CacheFocus §2.3.1: groups needed for n_docs caches."""
    per_group = max(1, window // doc_len)
    return (n_docs + per_group - 1) // per_group


def prune_layers(n_layers: int, every: int) -> list:
    """Layers (from 0) after which CacheFocus prunes (§2.4, every n-th layer):
    every-1, 2*every-1, ..."""
    return list(range(every - 1, n_layers, every)) if every >= 1 else []


def keep_schedule(n_docs: int, k_finish: int, n_layers: int, every: int) -> list:
    """Caches left after each pruning layer (CacheFocus App. C: (k - k_finish)
    / (L / n) removed per pruning layer).  The p-th of the P pruning layers
    leaves n_docs - floor(p * (n_docs - k_finish) / P), which is the page's
    count when it is whole and ends at k_finish in any case."""
    P = len(prune_layers(n_layers, every))
    return [n_docs - (p * (n_docs - k_finish)) // P for p in range(1, P + 1)]


def chunk_offsets(chunk_lens: Sequence[int]) -> list:
    """Delta_i of InfoFlow KV §4.2 (g(t) = Delta_i + p_i(t)): the global start of
    chunk i in the concatenated order."""
    out, acc = [], 0
    for n in chunk_lens:
        out.append(acc)
        acc += int(n)
    return out


def refill_budget(window: int, m: int, eta: int, interval: int) -> int:
    """ACRE §2.4 Eq. 17: L1 entries refilled, floor(min(W - m, eta) / l), never
    below zero."""
    room = min(window - m, eta)
    return room // interval if room > 0 else 0


def recompute_budget(n_tokens: int, ratio: str = "0.15") -> int:
    """InfoFlow KV §6.1: a fixed ratio of the context tokens, rounded down."""
    return int(Fraction(ratio) * n_tokens)


def delta_tensor(values: Sequence[int], device) -> torch.Tensor:
    return torch.tensor(list(values), dtype=torch.int64, device=device)
