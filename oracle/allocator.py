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
* Prefix caching ("PagedAttention" daily term, the prefix-caching paragraph
  after the copy-on-write figure; "Serving: vLLM and PagedAttention", section
  2.6): a full block is named by a hash chaining the parent block's hash, the
  block's token ids and extra keys, and a later request with the same prefix
  points at the cached blocks. Readings: the hash is SHA-256 over parent (32
  zero bytes for the first block) || token ids as little-endian int32 ||
  extra; the longest run of leading cached blocks is reused; a freed block
  keeps its hash until the free list hands it out again, and reusing such a
  block takes it back off the free list.
"""

import hashlib
import struct


class NoBlocks(Exception):
    """The pool has fewer free blocks than the operation needs (nothing changed)."""


class TwinAllocator:
    def __init__(self, num_blocks, block_size):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("pool and block size must be positive")
        self.P = num_blocks
        self.bs = block_size
        self.ref = [0] * num_blocks
        self.seqs = {}                                    # id -> [blocks, length]
        # free list: a stack of (block, stamp); an entry counts only while the
        # block is free and the stamp is the block's latest (a cached block
        # taken back leaves a stale entry behind)
        self.stamp = [0] * num_blocks
        self.stack = []
        self.n_free = 0
        for b in range(num_blocks - 1, -1, -1):           # first pop -> 0
            self._push(b)
        self.cached = {}                                  # hash -> block
        self.hash_of = {}                                 # block -> hash
        self.hits = 0
        self.misses = 0

    @property
    def free(self):
        """The free blocks, in pop order reversed (last element pops first)."""
        return [b for b, st in self.stack if self.ref[b] == 0 and st == self.stamp[b]]

    def _push(self, b):
        self.stamp[b] += 1
        self.stack.append((b, self.stamp[b]))
        self.n_free += 1

    # -- sequence operations -------------------------------------------------
    def create(self, seq_id):
        if seq_id in self.seqs:
            raise KeyError(f"sequence {seq_id} exists")
        self.seqs[seq_id] = [[], 0]

    def _pop(self):
        while True:
            b, st = self.stack.pop()
            if self.ref[b] == 0 and st == self.stamp[b]:
                break
        self.ref[b] = 1
        self.n_free -= 1
        self._forget(b)                                   # its contents are about to change
        return b

    def _forget(self, b):
        h = self.hash_of.pop(b, None)
        if h is not None and self.cached.get(h) == b:
            del self.cached[h]

    def _remember(self, b, h):
        old = self.cached.get(h)
        if old is not None and old != b:
            self.hash_of.pop(old, None)
        self.cached[h] = b
        self.hash_of[b] = h

    def append(self, seq_id, n):
        """Append n token positions; returns (slots, cow_pairs)."""
        if n < 0:
            raise ValueError("negative token count")
        blocks, length = self.seqs[seq_id]
        bs = self.bs
        cow = n > 0 and length % bs != 0 and self.ref[blocks[-1]] > 1
        have = -(-length // bs)
        need = -(-(length + n) // bs) - have + (1 if cow else 0)
        if need > self.n_free:
            raise NoBlocks(f"need {need} blocks, {self.n_free} free")
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
                self._push(b)

    # -- prefix caching ----------------------------------------------------------
    @staticmethod
    def block_hashes(tokens, bs, extra=b""):
        """Chained hashes of the full blocks of a token sequence (list of 32-byte
        digests)."""
        out, parent = [], bytes(32)
        for k in range(len(tokens) // bs):
            block = tokens[k * bs:(k + 1) * bs]
            data = parent + struct.pack("<%di" % bs, *[int(t) for t in block]) + bytes(extra)
            parent = hashlib.sha256(data).digest()
            out.append(parent)
        return out

    def create_prefixed(self, seq_id, tokens, extra=b""):
        """New sequence holding a prompt; reuses the longest run of leading cached
        full blocks. Returns (slots, n_cached_tokens)."""
        if seq_id in self.seqs:
            raise KeyError(f"sequence {seq_id} exists")
        bs, n = self.bs, len(tokens)
        hs = self.block_hashes(tokens, bs, extra)
        hit_ids = []
        for h in hs:
            if h not in self.cached:
                break
            hit_ids.append(self.cached[h])
        hit = len(hit_ids)
        revive = sum(1 for b in hit_ids if self.ref[b] == 0)
        fresh = -(-n // bs) - hit
        if revive + fresh > self.n_free:
            raise NoBlocks(f"need {revive + fresh} blocks, {self.n_free} free")
        blocks = []
        for b in hit_ids:
            if self.ref[b] == 0:
                self.n_free -= 1                          # its stack entry goes stale
            self.ref[b] += 1
            blocks.append(b)
        for j in range(hit, -(-n // bs)):
            b = self._pop()
            if j < len(hs):
                self._remember(b, hs[j])
            blocks.append(b)
        self.seqs[seq_id] = [blocks, n]
        self.hits += hit
        self.misses += len(hs) - hit
        return [blocks[p // bs] * bs + p % bs for p in range(n)], hit * bs

    def prefix_stats(self):
        return {"hit_blocks": self.hits, "miss_blocks": self.misses, "cached_blocks": len(self.cached)}

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
        used = self.P - self.n_free
        slots = used * self.bs
        tokens = sum(fill.values())
        return {
            "num_blocks": self.P, "free_blocks": self.n_free, "used_blocks": used,
            "slots_allocated": slots, "tokens_stored": tokens,
            "waste": (1.0 - tokens / slots) if slots else 0.0,
        }
