"""Encoder-embedding block cache -- TEST INFRASTRUCTURE ONLY (part of the
oracle; see the package docstring).

What the AWS Neuron on-device encoder cache page describes ("Buffer Layout",
"Write Path", "Read Path", "Merge Inside Compiled Graph"):

* The cache is one preallocated buffer ``[num_blocks, block_size, fat_dim]``;
  each block holds one item's post-merger embeddings; the last block is a
  scratch block that takes the encoder's bucket-padding writes and is never
  given to an item.
* Write: the encoder's output blocks are scattered into the buffer at the
  block ids allocated for them (padding blocks go to the scratch block).
* Read/merge: the prefill takes the buffer, a block-id index ``[max_blocks]``
  and a position map ``[max_blocks, block_size]`` (int64) giving, for every
  token of every gathered block, its row in the batch's hidden states; the
  sentinel ``num_tokens`` marks a don't-care token, whose write lands in a
  dummy row that is thrown away.
* Fail loud: every scheduled position must have been filled.

Plain numpy and Python loops over blocks and tokens.
"""
from __future__ import annotations

from typing import Sequence, Tuple

import numpy as np


def write_blocks(buffer: np.ndarray, src: np.ndarray, block_ids: Sequence[int]) -> np.ndarray:
    """A copy of ``buffer`` with ``src[k]`` stored at block ``block_ids[k]``
    (ids outside the buffer are dropped)."""
    out = buffer.copy()
    for k, b in enumerate(block_ids):
        b = int(b)
        if 0 <= b < out.shape[0]:
            out[b] = src[k]
    return out


def merge_blocks(buffer: np.ndarray, block_ids: Sequence[int], positions: np.ndarray, hidden: np.ndarray,
                 num_tokens: int) -> np.ndarray:
    """A copy of ``hidden`` with token ``t`` of gathered block ``j`` written at
    row ``positions[j, t]`` when that row is real (``0 <= p < num_tokens``);
    sentinel and other out-of-range positions change nothing real.  Blocks
    whose id is outside the buffer contribute nothing."""
    out = hidden.copy()
    for j, b in enumerate(block_ids):
        b = int(b)
        if not 0 <= b < buffer.shape[0]:
            continue
        for t in range(positions.shape[1]):
            p = int(positions[j, t])
            if 0 <= p < num_tokens:
                out[p] = buffer[b, t]
    return out


def fill_counts(block_ids: Sequence[int], positions: np.ndarray, num_blocks: int, num_tokens: int) -> np.ndarray:
    """How many gathered tokens land on each real row."""
    cnt = np.zeros(num_tokens, np.int64)
    for j, b in enumerate(block_ids):
        if not 0 <= int(b) < num_blocks:
            continue
        for p in positions[j]:
            if 0 <= int(p) < num_tokens:
                cnt[int(p)] += 1
    return cnt


def check_filled(counts: np.ndarray, scheduled: np.ndarray = None) -> Tuple[int, int]:
    """(scheduled rows never written, rows written more than once)."""
    counts = np.asarray(counts)
    sched = np.ones(len(counts), bool) if scheduled is None else np.asarray(scheduled, bool)
    return int(np.sum(sched & (counts == 0))), int(np.sum(counts > 1))
