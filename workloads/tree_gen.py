"""Seeded synthetic inputs for building the draft tree from the last logits.

Recipe (one ``numpy.random.default_rng(seed)``), drawn in this order:
``history[B, cap]`` int32 uniform over a small alphabet ``[0, A)`` (so that
n-grams recur and both kinds of query find earlier occurrences, as in the
repetitive contexts retrieval drafting relies on), then ``logits[B, V]``
float32 N(0, 1) with ``boost`` added to the alphabet's entries (so the next
token and the guesses are tokens that occur in the history). bf16 cases round
the logits to bfloat16 (nearest, ties to even) and keep the bit patterns.
``history_len`` is given by the caller. This module draws numbers only; it
holds none of the tree-construction logic.
"""

from __future__ import annotations

import dataclasses
from typing import Sequence

import numpy as np

from .gen import bf16_bits_to_f32, f32_to_bf16_bits


@dataclasses.dataclass
class TreeCase:
    dtype: str
    B: int
    V: int
    history: np.ndarray      # int32 [B, cap]
    history_len: np.ndarray  # int32 [B]
    logits: np.ndarray       # float32 or uint16 bf16 bits [B, V]

    def logits_f64(self) -> np.ndarray:
        if self.dtype == "bf16":
            return bf16_bits_to_f32(self.logits).astype(np.float64)
        return self.logits.astype(np.float64)


def make_tree_case(*, B: int, V: int, cap: int, history_len: Sequence[int], alphabet: int = 16,
                   boost: float = 5.0, dtype: str = "bf16", seed: int = 0) -> TreeCase:
    rng = np.random.default_rng(seed)
    hist = rng.integers(0, alphabet, size=(B, cap)).astype(np.int32)
    logits = rng.standard_normal((B, V), dtype=np.float32)
    logits[:, :min(alphabet, V)] += np.float32(boost)
    if dtype == "bf16":
        logits = f32_to_bf16_bits(logits)
    return TreeCase(dtype=dtype, B=B, V=V, history=hist, history_len=np.asarray(history_len, dtype=np.int32),
                    logits=logits)
