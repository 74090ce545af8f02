"""Slot mapping: where a token at a given position of a sequence is stored.

Test infrastructure only (see the package docstring).

Position p of a sequence (0-based) is in logical block p // bs at offset p % bs;
the block table maps the logical block to a physical block ("03 ·
PagedAttention", "Blocks and block tables": the table from logical block to
physical block, tokens 0-15 in logical block 0 and so on; "Serving: vLLM and
PagedAttention", section 2.2). The flat slot is physical_block * bs + offset.
"""

import numpy as np


def slots_for_positions(block_tables, positions, bs):
    """int64[S]: slot of token ``positions[i]`` of sequence i (-1 where position < 0)."""
    out = np.full(len(positions), -1, dtype=np.int64)
    for i, p in enumerate(positions):
        p = int(p)
        if p < 0:
            continue
        block = int(block_tables[i][p // bs])
        if block < 0:
            raise ValueError("position beyond the allocated blocks")
        out[i] = block * bs + p % bs
    return out


def decode_slots(block_tables, context_lens, bs):
    """int64[S]: slot of the newest token of each sequence, at position L_i - 1.

    The context length includes the token being written this step; a sequence
    with L_i <= 0 writes nothing (slot -1).
    """
    return slots_for_positions(block_tables, [int(L) - 1 for L in context_lens], bs)
