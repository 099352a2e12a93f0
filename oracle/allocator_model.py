"""Block-pool allocator, plain Python -- test infrastructure (oracle side).

Behaviour follows the block manager of "Reducing LLM Inference Latency: KV
Cache Quantization and PagedAttention in vLLM" (section "PagedAttention:
Solving VRAM Fragmentation", the block-manager emulation): a FIFO free list
of physical block ids, allocate takes ceil(n / p) blocks from its front,
free returns a sequence's blocks to its back in table order, and token t of
a sequence sits in physical block table[t // p] at offset t % p.  Appending
follows the BlockTable of "Optimizing LLM Inference: KV Cache and
PagedAttention Explained" (section "PagedAttention: Operating Systems to the
Rescue"): a new block is taken only when the token count is a multiple of
p.  Prefix sharing ("KV Cache Compression & Paged Attention Deep Dive",
section "PagedAttention: Operating System-Inspired Memory Management")
points several tables at the same physical blocks; reference counts decide
when a block returns to the free list.

Readings where the pages are silent or inconsistent:

* every operation is all-or-nothing: exhaustion raises before any block is
  taken (the emulation pops blocks one by one and leaks them on failure);
* allocating an existing sequence is an error (the emulation overwrites);
* copy-on-write, which "KV Cache Compression & Paged Attention Deep Dive"
  (sections "PagedAttention: Operating System-Inspired Memory Management" and
  "Implementation Details: PagedAttention Kernel and Page Table") names
  together with per-block reference counts but does not spell out, is read
  as follows: a fork may end anywhere inside the source, and the new
  sequence shares every block that holds part of its prefix, the last one
  possibly partly filled.  A sequence about to write into a partly filled
  block that another table also points at first takes a fresh block from
  the front of the free list, records the copy (old block -> new block) and
  points its table at the new block, dropping one reference to the old one.
  That block is taken before any block the append itself needs.
* automatic prefix caching ("KV Cache Compression & Paged Attention Deep
  Dive", section "Implementation Details: PagedAttention Kernel and Page
  Table": the prefix is hashed and a cached block is looked up before new
  ones are allocated; "KV Cache Optimization: 3x Faster LLM Inference on
  24GB VRAM", section "Prefix Caching: The Hidden Multiplier": later
  requests reuse the pages of a common prefix, and pages are evicted in
  LRU order) is read as follows.  Every full block of a prompt allocated
  with token ids is entered in a cache under the key (the cache entry of
  the block before it, or none for the first block; the block's p token
  ids), compared exactly, so a hash collision cannot produce a false hit.
  Entry ids are never reused, so the entries below an evicted block become
  unreachable.  A new prompt walks its full blocks in order and reuses
  every block found, stopping at the first miss; the count of reused
  tokens is returned so that only the rest is computed and written.  A
  cached block whose last reference is dropped is not freed: it joins an
  LRU list and can still be found.  Blocks are taken from the free list
  first; when it is empty, the least recently released cached block is
  evicted (its entry removed) and taken.  Blocks filled by later appends
  carry no token ids and are not cached.
* swapping ("Reducing LLM Inference Latency: KV Cache Quantization and
  PagedAttention in vLLM", section "Prefill Swapping and GPU Thrashing":
  when the pool is exhausted, blocks are allocated in host memory and KV
  pages are moved there over PCIe; the number of swapped requests is a
  metric) is read as follows.  A pool may have a second FIFO of host
  blocks.  Swapping a sequence out moves every block it holds alone
  (reference count 1) to a host block taken from the front of the host
  FIFO, in table order, and releases the device block; blocks another
  table also points at keep their device reference.  Swapping in takes a
  device block for each host entry, in table order, and returns the host
  blocks to the back of the host FIFO.  A swapped sequence can only be
  swapped in or freed.  Both are all-or-nothing and refused while copies
  are pending.  Each returns its (device block, host block) pairs for the
  caller to move the data: out before any later write to the pool, in
  before the sequence is read.
* recorded copies stay pending until the caller takes them and runs them on
  the device, before the tokens of the same appends are written.  While any
  is pending, fork and free are refused: with no fork a copy's destination
  is never shared (so never copied from), and with no free neither end of a
  pending copy returns to the free list, so the copies of one batch never
  overlap and may run in parallel.
"""
from __future__ import annotations

import collections
from typing import Dict, List, Optional, Sequence, Tuple


class OutOfBlocks(MemoryError):
    pass


class AllocatorError(ValueError):
    pass


class CopiesPending(AllocatorError):
    pass


class Swapped(AllocatorError):
    pass


class BlockPoolModel:
    def __init__(self, num_blocks: int, block_size: int,
                 free_order: Optional[Sequence[int]] = None):
        if num_blocks <= 0 or block_size <= 0:
            raise AllocatorError("num_blocks and block_size must be positive")
        order = list(range(num_blocks)) if free_order is None else [int(x) for x in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise AllocatorError("free_order must be a permutation of 0..num_blocks-1")
        self.num_blocks = num_blocks
        self.p = block_size
        self.free = collections.deque(order)
        self.ref = [0] * num_blocks
        self.tables: Dict[int, List[int]] = {}
        self.ntok: Dict[int, int] = {}
        self.copies: List[Tuple[int, int]] = []
        # prefix cache: key -> block, block -> (entry id, key), evictable LRU
        self.cache: Dict[tuple, int] = {}
        self.entry: Dict[int, Tuple[int, tuple]] = {}
        self.lru: "collections.OrderedDict[int, None]" = collections.OrderedDict()
        self.next_entry = 0
        self.hits = 0      # blocks found by lookups
        self.queries = 0   # full blocks looked up
        # host blocks for swapping: FIFO of free host block ids; per swapped
        # sequence, which table entries are host blocks
        self.host_free: "collections.deque[int]" = collections.deque()
        self.num_host_blocks = 0
        self.on_host: Dict[int, List[bool]] = {}

    def set_host_blocks(self, n: int) -> None:
        if self.num_host_blocks - len(self.host_free) > 0:
            raise AllocatorError("host blocks in use")
        self.num_host_blocks = n
        self.host_free = collections.deque(range(n))

    def _live(self, seq: int) -> None:
        if seq not in self.tables:
            raise AllocatorError("no such sequence")
        if seq in self.on_host:
            raise Swapped("sequence is swapped out")

    def swap_out(self, seq: int) -> List[Tuple[int, int]]:
        self._live(seq)
        if self.copies:
            raise CopiesPending("copies pending")
        table = self.tables[seq]
        move = [i for i, b in enumerate(table) if self.ref[b] == 1]
        if len(move) > len(self.host_free):
            raise OutOfBlocks("host block pool exhausted")
        flags = [False] * len(table)
        pairs = []
        for i in move:
            h = self.host_free.popleft()
            pairs.append((table[i], h))
            self._release(table[i])
            table[i] = h
            flags[i] = True
        self.on_host[seq] = flags
        return pairs

    def swap_in(self, seq: int) -> List[Tuple[int, int]]:
        if seq not in self.tables:
            raise AllocatorError("no such sequence")
        if seq not in self.on_host:
            raise AllocatorError("sequence is not swapped out")
        if self.copies:
            raise CopiesPending("copies pending")
        table, flags = self.tables[seq], self.on_host[seq]
        idx = [i for i, f in enumerate(flags) if f]
        new = self._take(len(idx))
        pairs = []
        for i, b in zip(idx, new):
            pairs.append((b, table[i]))
            self.host_free.append(table[i])
            table[i] = b
        del self.on_host[seq]
        return pairs

    def swap_stats(self):
        """(swapped sequences, free host blocks, used host blocks)."""
        free = len(self.host_free)
        return len(self.on_host), free, self.num_host_blocks - free

    # -- operations -------------------------------------------------------
    def available(self) -> int:
        """Blocks an allocation can take: free ones and evictable cached ones."""
        return len(self.free) + len(self.lru)

    def _take(self, k: int) -> List[int]:
        if k > self.available():
            raise OutOfBlocks("block pool exhausted")
        out = []
        for _ in range(k):
            if self.free:
                b = self.free.popleft()
            else:  # evict the least recently released cached block
                b, _ = self.lru.popitem(last=False)
                _, key = self.entry.pop(b)
                del self.cache[key]
            self.ref[b] = 1
            out.append(b)
        return out

    def _release(self, b: int) -> None:
        """Drop one reference; at zero a cached block becomes evictable and
        any other block returns to the back of the free list."""
        self.ref[b] -= 1
        if self.ref[b] == 0:
            if b in self.entry:
                self.lru[b] = None
            else:
                self.free.append(b)

    def _lookup(self, tokens: Sequence[int]) -> List[int]:
        """Cached blocks matching the prompt's leading full blocks."""
        found, parent = [], -1
        for i in range(len(tokens) // self.p):
            key = (parent, tuple(int(t) for t in tokens[i * self.p:(i + 1) * self.p]))
            b = self.cache.get(key)
            if b is None:
                break
            found.append(b)
            parent = self.entry[b][0]
        return found

    def allocate_cached(self, seq: int, tokens: Sequence[int]) -> int:
        """New sequence holding the prompt `tokens`; reuses cached blocks of
        its leading full blocks.  Returns the number of reused tokens."""
        if seq in self.tables:
            raise AllocatorError("sequence exists")
        if seq < 0:
            raise AllocatorError("sequence ids are >= 0")
        n = len(tokens)
        found = self._lookup(tokens)
        need = -(-n // self.p) - len(found)
        revive = sum(1 for b in found if self.ref[b] == 0)
        if need > self.available() - revive:
            raise OutOfBlocks("block pool exhausted")
        self.queries += n // self.p
        self.hits += len(found)
        for b in found:
            if self.ref[b] == 0:
                del self.lru[b]
            self.ref[b] += 1
        table = found + self._take(need)
        parent = self.entry[found[-1]][0] if found else -1
        for i in range(len(found), n // self.p):
            key = (parent, tuple(int(t) for t in tokens[i * self.p:(i + 1) * self.p]))
            self.cache[key] = table[i]
            self.entry[table[i]] = (self.next_entry, key)
            parent = self.next_entry
            self.next_entry += 1
        self.tables[seq] = table
        self.ntok[seq] = n
        return len(found) * self.p

    def allocate(self, seq: int, n: int) -> None:
        if seq in self.tables:
            raise AllocatorError("sequence exists")
        if n < 0:
            raise AllocatorError("negative token count")
        self.tables[seq] = self._take(-(-n // self.p))
        self.ntok[seq] = n

    def _needs_copy(self, seq: int, k: int) -> bool:
        """True when the next token of seq lands in a partly filled block
        that another table also points at."""
        n = self.ntok[seq]
        return k > 0 and n % self.p != 0 and self.ref[self.tables[seq][-1]] > 1

    def append(self, seq: int, k: int) -> List[int]:
        """Add k tokens; returns their slots."""
        self._live(seq)
        if k < 0:
            raise AllocatorError("negative token count")
        n = self.ntok[seq]
        table = self.tables[seq]
        cow = self._needs_copy(seq, k)
        grow = max(-(-(n + k) // self.p) - len(table), 0)
        if grow + cow > self.available():
            raise OutOfBlocks("block pool exhausted")
        if cow:
            old = table[-1]
            table[-1] = self._take(1)[0]
            self.ref[old] -= 1  # still held by another table
            self.copies.append((old, table[-1]))
        table.extend(self._take(grow))
        self.ntok[seq] = n + k
        return [self.slot(seq, t) for t in range(n, n + k)]

    def take_copies(self) -> List[Tuple[int, int]]:
        """Pending (source block, destination block) copies, in the order
        they were recorded; the list is emptied."""
        out, self.copies = self.copies, []
        return out

    def fork(self, src: int, dst: int, prefix_tokens: int) -> None:
        self._live(src)
        if dst in self.tables:
            raise AllocatorError("sequence exists")
        if dst < 0:
            raise AllocatorError("sequence ids are >= 0")
        if prefix_tokens > self.ntok[src] or prefix_tokens < 0:
            raise AllocatorError("fork length outside the source")
        if self.copies:
            raise CopiesPending("copies pending")
        shared = self.tables[src][: -(-prefix_tokens // self.p)]
        for b in shared:
            self.ref[b] += 1
        self.tables[dst] = list(shared)
        self.ntok[dst] = prefix_tokens

    def free_seq(self, seq: int) -> None:
        if seq not in self.tables:
            raise AllocatorError("no such sequence")
        if self.copies:
            raise CopiesPending("copies pending")
        flags = self.on_host.pop(seq, None)
        for i, b in enumerate(self.tables.pop(seq)):
            if flags and flags[i]:
                self.host_free.append(b)
            else:
                self._release(b)
        del self.ntok[seq]

    # -- queries ----------------------------------------------------------
    def physical_address(self, seq: int, t: int):
        self._live(seq)
        if not (0 <= t < self.ntok[seq]):
            raise AllocatorError("bad token index")
        return self.tables[seq][t // self.p], t % self.p

    def slot(self, seq: int, t: int) -> int:
        blk, off = self.physical_address(seq, t)
        return blk * self.p + off

    def stats(self):
        """(free, used, usage): evictable cached blocks count as free."""
        free = self.available()
        used = self.num_blocks - free
        return free, used, used / self.num_blocks

    def cache_stats(self):
        """(cached blocks, evictable cached blocks, block hits, blocks looked up)."""
        return len(self.entry), len(self.lru), self.hits, self.queries

    def block_tables(self, seqs: Sequence[int], width: int):
        import numpy as np

        bt = np.full((len(seqs), width), -1, dtype=np.int32)
        cl = np.zeros(len(seqs), dtype=np.int32)
        for i, s in enumerate(seqs):
            self._live(s)
            row = self.tables[s]
            if len(row) > width:
                raise AllocatorError("table width too small")
            bt[i, : len(row)] = row
            cl[i] = self.ntok[s]
        return bt, cl

    def run_ops(self, ops) -> None:
        """Execute a workload's allocation operations."""
        for op in ops:
            if op[0] == "allocate":
                self.allocate(op[1], op[2])
            elif op[0] == "fork":
                self.fork(op[1], op[2], op[3])
            elif op[0] == "append":
                self.append(op[1], op[2])
            else:
                raise ValueError(op)
