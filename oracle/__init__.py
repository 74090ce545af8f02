"""Plain, slow, fp64 CPU oracle for paged decode attention and the KV-cache write.

This package is TEST INFRASTRUCTURE. It is what the GPU path is checked
against, never part of it: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything here. The
product path (the ``paged_kv_cache_108_amd`` package and its HIP library)
neither imports this package nor shares any code, table or helper with it.

Every function is written from the pages' statement of what is computed:

* "03 · PagedAttention" (sunilkunchoor.github.io): sections "Blocks and block
  tables", "Why this eliminates the waste, precisely", "Sharing: copy-on-write",
  "Try It / Experiment 1" and the block-size table under "Now change one thing".
* "PagedAttention" daily term (mlapandio.dev): the decode-step figure, the
  copy-on-write figure, "Pros" ("not an approximation"), "Cons", and the
  capacity-math example.
* "paged-attention" lesson (tbash.cc): the five-request worked example and the
  statement that the output is identical whatever the layout.
* "Serving: vLLM and PagedAttention" (henryfzh-note.com): section 2.2 (block
  table, last-block fill, tail-waste arithmetic); sections 2.4 and 2.7 (windows
  of several new queries over the same cache: ``paged_multi_query_attn``).
* Shared prefix blocks ("03 · PagedAttention", "Sharing: copy-on-write"):
  ``paged_decode_lse`` and ``merge_attn_states`` give the state of an attention
  over part of a sequence and the exact combination of two such parts.

The attention itself is the textbook definition applied to the sequence's
K/V reassembled in logical order: the pages state that paging changes only the
layout, never the result, so the oracle is that definition written out in
float64 with numpy.

Pinning. Each function is pinned by ``tests/test_oracle_*.py`` to something
other than itself: numbers the pages print (``tests/golden``), closed forms,
invariants the pages state, a library routine on tiny inputs, brute force.
"""

from .codecs import (bf16_bits_to_f64, f32_to_f64, e4m3_value_table, e4m3_decode,
                     e4m3_encode)
from .attention import (reassemble, paged_decode_attn, contiguous_decode_attn, paged_multi_query_attn,
                        contiguous_decode_lse, paged_decode_lse, merge_attn_states)
from .cache_write import kv_cache_write, quantise, copy_blocks
from .slots import decode_slots, slots_for_positions
from .waste import (blocks_for, paged_slots, naive_slots, tail_slots, utilisation,
                    waste_fraction, capacity)
from .allocator import TwinAllocator, NoBlocks
from .splitk import partition_then_merge

__all__ = [
    "bf16_bits_to_f64", "f32_to_f64", "e4m3_value_table", "e4m3_decode", "e4m3_encode",
    "reassemble", "paged_decode_attn", "contiguous_decode_attn", "paged_multi_query_attn",
    "contiguous_decode_lse", "paged_decode_lse", "merge_attn_states",
    "kv_cache_write", "quantise",
    "copy_blocks",
    "decode_slots", "slots_for_positions", "blocks_for", "paged_slots",
    "naive_slots", "tail_slots", "utilisation", "waste_fraction", "capacity",
    "TwinAllocator", "NoBlocks", "partition_then_merge",
]
