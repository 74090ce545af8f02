"""Allocation and tail-waste arithmetic of a paged KV cache.

Test infrastructure only (see the package docstring).

* A sequence of L tokens holds ceil(L / bs) blocks: a new block is taken only
  when the previous one is full ("03 · PagedAttention", "Blocks and block
  tables"; "Check Yourself": the worst case is bs*ceil(L/bs) - L <= bs - 1
  wasted slots).
* The unfilled tail of the last block is the only waste: (bs - L mod bs) mod bs
  slots ("Serving: vLLM and PagedAttention", section 2.2, read with the mod-0
  case fixed; "paged-attention" lesson, tail-waste column).
* Waste is 1 - used / allocated and utilisation used / allocated (the
  "paged-attention" lesson computes waste that way; "03 · PagedAttention",
  Experiment 1 prints utilisation as stored / allocated).
* A naive allocator reserves max_len slots per request (the lesson's
  reserve-max comparator; "03 · PagedAttention", "The Problem").
* Capacity of a pool is floor(pool_slots / (allocated / n)): the lesson's
  requests-per-pool comparison.
"""

import numpy as np


def blocks_for(L, bs):
    """Blocks a sequence of L tokens occupies (0 for L <= 0)."""
    L = np.asarray(L, dtype=np.int64)
    return np.where(L > 0, -(-L // bs), 0)


def tail_slots(L, bs):
    """Unfilled slots in the last block."""
    return blocks_for(L, bs) * bs - np.maximum(np.asarray(L, dtype=np.int64), 0)


def paged_slots(lengths, bs):
    """Total slots a paged allocator hands out for these lengths."""
    return int(np.sum(blocks_for(lengths, bs) * bs))


def naive_slots(lengths, max_len):
    """Total slots reserved when every request reserves max_len up front."""
    return int(len(lengths) * max_len)


def utilisation(lengths, allocated):
    return float(np.sum(np.asarray(lengths, dtype=np.int64))) / float(allocated)


def waste_fraction(lengths, allocated):
    return 1.0 - utilisation(lengths, allocated)


def capacity(pool_slots, allocated, n):
    """Requests of this mix that fit a pool: floor(pool / (allocated / n))."""
    return int(np.floor(pool_slots / (allocated / n)))
