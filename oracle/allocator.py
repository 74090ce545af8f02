"""A plain-Python twin of the host block allocator (free list, refcounts, CoW).

Test infrastructure only (see the package docstring). The library's C++
allocator must produce the same block tables, slots and copy-on-write pairs as
this twin for the same sequence of operations.

What the pages fix, and the readings taken where they leave a choice:

* The pool is a fixed set of P equal blocks, all allocated at start; any free
  block fits any request, so the allocator is a plain free list with no search
  ("03 · PagedAttention", "Blocks and block tables"; "PagedAttention" daily
  term, "Pros"). Reading: a LIFO stack whose first pop returns block 0.
* A block is taken only when a sequence's previous block is full: the 17th
  token takes a new block, tokens 18-32 take none ("03 · PagedAttention",
  "Blocks and block tables" and "Check Yourself").
* Sharing: a fork points the child's table at the parent's blocks and raises
  each block's reference count ("03 · PagedAttention", "Sharing: copy-on-write";
  "PagedAttention" daily term, copy-on-write figure).
* Copy-on-write: a write into a block whose count is above one first copies the
  block, repoints the writer's entry at the copy and lowers the original's count
  by one ("03 · PagedAttention", "Sharing: copy-on-write"). Reading: it fires
  when tokens are appended into a shared, partially filled last block (the
  daily term's figure: "the shared block is not full"); the (src, dst) pair is
  reported so the caller can copy the data.
* Exhaustion is not a failure of the allocator: the scheduler preempts
  ("03 · PagedAttention", "When the pool runs dry"). Reading: an append that
  needs more blocks than are free changes nothing and reports NoBlocks.
* Freeing lowers every block's count, last logical block first, and returns a
  block to the free list when its count reaches zero.
"""


class NoBlocks(Exception):
    """The pool has fewer free blocks than the operation needs (nothing changed)."""


class TwinAllocator:
    def __init__(self, num_blocks, block_size):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("pool and block size must be positive")
        self.P = num_blocks
        self.bs = block_size
        self.free = list(range(num_blocks - 1, -1, -1))   # pop() -> 0 first
        self.ref = [0] * num_blocks
        self.seqs = {}                                    # id -> [blocks, length]

    # -- sequence operations -------------------------------------------------
    def create(self, seq_id):
        if seq_id in self.seqs:
            raise KeyError(f"sequence {seq_id} exists")
        self.seqs[seq_id] = [[], 0]

    def _pop(self):
        b = self.free.pop()
        self.ref[b] = 1
        return b

    def append(self, seq_id, n):
        """Append n token positions; returns (slots, cow_pairs)."""
        if n < 0:
            raise ValueError("negative token count")
        blocks, length = self.seqs[seq_id]
        bs = self.bs
        cow = n > 0 and length % bs != 0 and self.ref[blocks[-1]] > 1
        have = -(-length // bs)
        need = -(-(length + n) // bs) - have + (1 if cow else 0)
        if need > len(self.free):
            raise NoBlocks(f"need {need} blocks, {len(self.free)} free")
        pairs = []
        if cow:
            src = blocks[-1]
            dst = self._pop()
            self.ref[src] -= 1
            blocks[-1] = dst
            pairs.append((src, dst))
        slots = []
        for p in range(length, length + n):
            j = p // bs
            if j == len(blocks):
                blocks.append(self._pop())
            slots.append(blocks[j] * bs + p % bs)
        self.seqs[seq_id][1] = length + n
        return slots, pairs

    def fork(self, parent, child):
        if parent not in self.seqs:
            raise KeyError(f"sequence {parent} not found")
        if child in self.seqs:
            raise KeyError(f"sequence {child} exists")
        blocks, length = self.seqs[parent]
        for b in blocks:
            self.ref[b] += 1
        self.seqs[child] = [list(blocks), length]

    def release(self, seq_id):
        blocks, _ = self.seqs.pop(seq_id)
        for b in reversed(blocks):
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)

    # -- views -----------------------------------------------------------------
    def tables(self, seq_ids, max_blocks):
        """(tables [S][max_blocks] padded with -1, lengths [S])."""
        tabs, lens = [], []
        for s in seq_ids:
            blocks, length = self.seqs[s]
            if len(blocks) > max_blocks:
                raise ValueError("table wider than max_blocks")
            tabs.append(list(blocks) + [-1] * (max_blocks - len(blocks)))
            lens.append(length)
        return tabs, lens

    def stats(self):
        """dict: num/free/used blocks, slots allocated, tokens stored, waste.

        A physical block shared by several tables holds the same prefix tokens,
        so its fill is the largest fill any table gives it.
        """
        fill = {}
        for blocks, length in self.seqs.values():
            for j, b in enumerate(blocks):
                f = min(self.bs, length - j * self.bs)
                fill[b] = max(fill.get(b, 0), f)
        used = self.P - len(self.free)
        slots = used * self.bs
        tokens = sum(fill.values())
        return {
            "num_blocks": self.P, "free_blocks": len(self.free), "used_blocks": used,
            "slots_allocated": slots, "tokens_stored": tokens,
            "waste": (1.0 - tokens / slots) if slots else 0.0,
        }
