"""Seeded inputs for the encoder-embedding block cache (the AWS Neuron
on-device encoder cache notes): which blocks the encoder's output goes to,
which blocks a prefill gathers, and where each gathered token lands.
Inputs only: no cache arithmetic.

Default geometry is the notes' Qwen3-VL one: 512 post-merger tokens per
block, fat_dim 20480 (bf16), 32 item blocks plus the scratch block; the
encoder writes a bucket of 8 output blocks (the last two padding, sent to
the scratch block); the prefill gathers 8 blocks (the 6 just written and 2
cached ones), each holding 256..512 real tokens (an image is 256), placed
on distinct rows of a 8192-token batch; every other token is the sentinel."""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass
class EncCacheCase:
    num_blocks: int       # including the scratch block (the last)
    block_size: int
    fat_dim: int
    write_ids: np.ndarray  # int32 [n_write]; padding blocks carry the scratch id
    gather_ids: np.ndarray  # int32 [max_blocks]
    positions: np.ndarray  # int64 [max_blocks, block_size]; num_tokens = sentinel
    num_tokens: int
    value_seed: int

    @property
    def scratch(self) -> int:
        return self.num_blocks - 1

    @property
    def real_tokens(self) -> int:
        return int(np.sum(self.positions < self.num_tokens))


def enc_cache_case(seed: int = 0, num_blocks: int = 33, block_size: int = 512, fat_dim: int = 20480,
                   n_write: int = 8, n_pad: int = 2, n_cached: int = 2, num_tokens: int = 8192,
                   token_range=(256, 512)) -> EncCacheCase:
    rng = np.random.default_rng([38, 7, seed])
    free = rng.permutation(num_blocks - 1)
    n_real = n_write - n_pad
    written = free[:n_real]
    cached = free[n_real:n_real + n_cached]
    write_ids = np.concatenate([written, np.full(n_pad, num_blocks - 1)]).astype(np.int32)
    gather_ids = rng.permutation(np.concatenate([written, cached])).astype(np.int32)
    m = len(gather_ids)
    counts = rng.integers(token_range[0], token_range[1] + 1, size=m)
    assert counts.sum() <= num_tokens
    rows = rng.permutation(num_tokens)
    pos = np.full((m, block_size), num_tokens, np.int64)
    k = 0
    for j in range(m):
        c = int(min(counts[j], block_size))
        pos[j, :c] = rows[k:k + c]
        k += c
    return EncCacheCase(num_blocks, block_size, fat_dim, write_ids, gather_ids, pos, num_tokens,
                        int(rng.integers(1 << 30)))
