"""Algorithmic byte and flop counts for paged decode attention.

These are the numerators of the bench's throughput and roofline figures.

- Block footprint, from the asynchronous-KV-prefetch review, section 4.2:
  M_block = b * d_h * T_block (bytes per element, head dim, tokens per block).
- Cache working set of one iteration, same section:
  M_total = M_block * (N_thread / 32) * H * B, i.e. one block per warp of every
  thread block, one thread block per head, for each of B sequences.
- Decode KV read volume, from the KV-cache-prefetching article, section 1.1:
  2 (K and V) * layers * kv_heads * head_dim * context * bytes per element.
  The per-layer form with a ragged batch replaces context by the sum of the
  context lengths: every KV token is read once per KV head.
"""
from __future__ import annotations

from typing import Iterable

FP16_BYTES = 2
HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published peak


def block_bytes(elem_bytes: int = FP16_BYTES, head_dim: int = 128,
                block_size: int = 16) -> int:
    """M_block: bytes of one (block, head) slice of K (or of V)."""
    return elem_bytes * head_dim * block_size


def iteration_working_set(block: int, n_thread: int, heads: int, batch: int,
                          warp: int = 32) -> int:
    """M_total: bytes of the blocks all warps touch in one loop iteration."""
    return block * (n_thread // warp) * heads * batch


def max_batch_in_cache(cache_bytes: int, block: int, n_thread: int, heads: int,
                       warp: int = 32) -> int:
    """Largest batch whose per-iteration working set fits the cache."""
    return cache_bytes // iteration_working_set(block, n_thread, heads, 1, warp)


def decode_kv_bytes(layers: int, kv_heads: int, head_dim: int, context: int,
                    elem_bytes: int = FP16_BYTES) -> int:
    """KV bytes one decode step reads for one sequence over all layers."""
    return 2 * layers * kv_heads * head_dim * context * elem_bytes


def step_kv_bytes(kv_heads: int, head_dim: int, context_lens: Iterable[int],
                  elem_bytes: int = FP16_BYTES) -> int:
    """KV bytes of one layer's decode attention over a batch (the bench's
    algorithmic volume; contexts <= 0 read nothing)."""
    total = sum(max(0, int(c)) for c in context_lens)
    return decode_kv_bytes(1, kv_heads, head_dim, total, elem_bytes)


def step_other_bytes(num_seqs: int, q_heads: int, head_dim: int,
                     context_lens: Iterable[int], block_size: int = 16,
                     elem_bytes: int = FP16_BYTES) -> int:
    """Q read, output written, block-table entries and context lengths read."""
    blocks = sum(-(-max(0, int(c)) // block_size) for c in context_lens)
    return 2 * num_seqs * q_heads * head_dim * elem_bytes + 4 * blocks + 4 * num_seqs


def step_flops(q_heads: int, head_dim: int, context_lens: Iterable[int]) -> int:
    """2*D for q.k plus 2*D for p*v, per query head and token."""
    total = sum(max(0, int(c)) for c in context_lens)
    return 4 * head_dim * q_heads * total
