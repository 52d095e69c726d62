"""Packing a padded batch into the cumulative-length layout, plain numpy.

TEST INFRASTRUCTURE: only tests, the smoke entry and the benchmark's CPU
baseline may import this module. The product path never does.

What it computes. DisentangledFlash's packed unpadded inference (README,
"Packed unpadded inference") takes right-padded hidden states and their
attention mask, keeps only the valid token rows, and describes the result
with int32 cumulative sequence lengths, FlashAttention style (fold-attention
README, packed self-attention): sequence b owns packed rows cu[b] ..
cu[b+1]-1. After attention the packed outputs go back to the padded layout,
with zero rows where the mask is zero. Kernels-community discussion #31
notes that packing pays where padding dominates (the MNLI run: 92.62%
padding) and costs a copy where it does not.

The packing metadata, for a [B, L] mask m (nonzero = valid):
  cu_seqlens[0] = 0, cu_seqlens[b+1] = cu_seqlens[b] + (number of valid l in row b)
  token_rows[r]   = the padded row index b*L + l of the r-th valid token in
                    row-major order (b first, then l), for r < cu[B]; -1 after
  row_to_packed[i] = r when token_rows[r] = i, else -1   (i < B*L)
and the two copies
  pack:   out[r] = src[token_rows[r]]          for r < cu[B]
  unpack: out[i] = src[row_to_packed[i]] if row_to_packed[i] >= 0 else 0

With a right-padded mask (the pages' case) the r-th token of sequence b sits
at position r - cu[b], so packed attention sees the padded positions. With
holes in the mask the valid tokens are still gathered in order; positions
then differ from the padded indices (the forward's padded entry keeps the
padded indices).
"""

from __future__ import annotations

import numpy as np


def pack_index(mask: np.ndarray | None, B: int, L: int):
    """Return (cu_seqlens int64[B+1], token_rows int64[B*L], row_to_packed
    int64[B*L]) for a [B, L] mask (None: every token valid)."""
    if mask is None:
        valid = np.ones((B, L), dtype=bool)
    else:
        valid = np.asarray(mask).reshape(B, L) != 0
    counts = valid.sum(axis=1).astype(np.int64)
    cu = np.zeros(B + 1, dtype=np.int64)
    cu[1:] = np.cumsum(counts)
    total = int(cu[-1])
    rows = np.flatnonzero(valid.reshape(-1)).astype(np.int64)   # row-major order
    token_rows = np.full(B * L, -1, dtype=np.int64)
    token_rows[:total] = rows
    row_to_packed = np.full(B * L, -1, dtype=np.int64)
    row_to_packed[rows] = np.arange(total, dtype=np.int64)
    return cu, token_rows, row_to_packed


def pack_rows(src: np.ndarray, token_rows: np.ndarray, total: int) -> np.ndarray:
    """[B*L, w] -> [total, w]: row r is src[token_rows[r]]."""
    return np.asarray(src)[np.asarray(token_rows)[:total]]


def unpack_rows(src: np.ndarray, row_to_packed: np.ndarray) -> np.ndarray:
    """[>= total, w] -> [B*L, w]: row i is src[row_to_packed[i]], or zeros."""
    src = np.asarray(src)
    idx = np.asarray(row_to_packed)
    out = np.zeros((idx.shape[0],) + src.shape[1:], dtype=src.dtype)
    keep = idx >= 0
    out[keep] = src[idx[keep]]
    return out
