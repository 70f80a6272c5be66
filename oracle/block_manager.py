"""Host block allocator model with reference counts and copy-on-write (TEST INFRASTRUCTURE, oracle).

[SMTS] "Paged KV-Cache with Radix Tree Prefix Cache" gives the allocator:
physical blocks carry a reference count; allocating a slot pops a block from
the free pool (the last element), increments its count and appends its id to
the sequence's list; an empty pool is an error that asks the scheduler to
preempt. Sequences sharing a prefix point at the same physical blocks through
copy-on-write pointers ([LLMI] interactive simulator, "copy-on-write prefix
caching").

Readings where the page is silent:
  * a pool of N blocks starts as the list [0, 1, ..., N-1], so the first
    allocation returns block N-1 (pop from the end); freed blocks are pushed
    back on the end in the sequence's logical order;
  * append_slot(seq) places the sequence's next token: at a block boundary it
    allocates a fresh block; otherwise it writes into the last block, and if
    that block is shared (ref_count > 1) it first allocates a private block,
    reports (src, dst) for a block copy, decrements the shared block's count
    and repoints the table entry;
  * fork(parent, child) shares every block of the parent (count + 1 each);
  * free(seq) decrements each of the sequence's blocks and returns those that
    reach zero to the pool;
  * on exhaustion nothing changes and OutOfBlocks is raised.

Swap ([LLMI] "9. Failure modes and limitations": a preempted request's KV
blocks are evicted to host memory and brought back later; [MTKV] "C++ Block
Scheduler and Asynchronous Fetch Kernel": blocks are demoted to pinned host
memory and promoted back to HBM with asynchronous copies). Readings:
  * swap_out(seq) returns the sequence's blocks in logical order (the caller
    copies them out before anything reuses them), then releases its
    references exactly as free() does; the sequence keeps its length and is
    marked swapped; shared blocks stay resident for the other sharers;
  * swap_in(seq) allocates cdiv(len, block_size) fresh blocks, popping them
    in logical order, and makes them the sequence's table; sharing is not
    restored (the copies are private); too few free blocks raise OutOfBlocks
    and change nothing;
  * a swapped sequence cannot append, fork or export its table; free() drops
    it.

Prefix cache ([LLMI] "8. Design Alternatives": a hash prefix cache over
16/32-token blocks, and an LRU radix tree over paged blocks; [SMTS] "Paged
KV-Cache with Radix Tree Prefix Cache": requests sharing a system prompt
reference the same physical blocks). Readings:
  * the cache is a radix tree whose nodes are full blocks, each keyed under
    its parent by its block_size token ids (exact: no hashing collisions);
  * match_prefix(seq, tokens) on a new sequence shares the longest chain of
    cached blocks that equals whole blocks of `tokens` (ref + 1 each) and
    makes them its table; it returns the number of tokens matched;
  * cache_prefix(seq, tokens) registers the sequence's first
    len(tokens) // block_size blocks under that chain; a block whose key is
    already cached (by another block) is left out, and so is everything after
    it;
  * a cached block whose count drops to 0 is not returned to the pool but
    becomes evictable; matching it again revives it;
  * allocation pops the free pool; when it is empty, the least recently used
    evictable block with no cached children is evicted (its key removed) and
    used instead; "use" is a match, a registration or a release to count 0,
    stamped from one counter;
  * num_free counts the pool only.
"""


class OutOfBlocks(MemoryError):
    pass


class BlockManagerModel:
    def __init__(self, num_blocks, block_size):
        self.block_size = block_size
        self.free_pool = list(range(num_blocks))
        self.ref = [0] * num_blocks
        self.tables = {}
        self.lens = {}
        self.swapped = set()
        self.node_of = {}        # cached block -> (parent block or None, token tuple)
        self.children = {}       # (parent block or None, token tuple) -> cached block
        self.n_children = {}     # cached block -> number of cached children
        self.stamp = {}          # cached block -> last use
        self.clock = 0

    def _tick(self, blk):
        self.clock += 1
        self.stamp[blk] = self.clock

    def _evictable(self):
        return [b for b in self.node_of if self.ref[b] == 0 and self.n_children[b] == 0]

    def _uncache(self, blk):
        parent, key = self.node_of.pop(blk)
        del self.children[(parent, key)]
        del self.n_children[blk]
        del self.stamp[blk]
        if parent is not None:
            self.n_children[parent] -= 1

    def _pop(self):
        if not self.free_pool:
            victims = self._evictable()
            if not victims:
                raise OutOfBlocks("KV block pool exhausted; preempt a sequence")
            blk = min(victims, key=lambda b: self.stamp[b])
            self._uncache(blk)
            self.ref[blk] += 1
            return blk
        blk = self.free_pool.pop()
        self.ref[blk] += 1
        return blk

    def _release(self, blk):
        self.ref[blk] -= 1
        if self.ref[blk] == 0:
            if blk in self.node_of:
                self._tick(blk)              # evictable, keeps its data and key
            else:
                self.free_pool.append(blk)

    def match_prefix(self, seq, tokens):
        """Share the longest cached chain of whole blocks of `tokens` with a new sequence."""
        if seq in self.tables or seq in self.swapped:
            raise KeyError("match_prefix needs a new sequence")
        bs = self.block_size
        parent, blocks = None, []
        for i in range(len(tokens) // bs):
            blk = self.children.get((parent, tuple(tokens[i * bs:(i + 1) * bs])))
            if blk is None:
                break
            blocks.append(blk)
            parent = blk
        for blk in blocks:
            self.ref[blk] += 1
            self._tick(blk)
        self.tables[seq] = blocks
        self.lens[seq] = len(blocks) * bs
        return len(blocks) * bs

    def cache_prefix(self, seq, tokens):
        """Register the sequence's first len(tokens) // block_size blocks in the cache."""
        if seq not in self.tables:
            raise KeyError("cache_prefix needs a resident sequence")
        bs = self.block_size
        n = len(tokens) // bs
        table = self.tables[seq]
        if n > len(table) or n * bs > self.lens[seq]:
            raise ValueError("more tokens than the sequence holds")
        parent = None
        for i in range(n):
            key = (parent, tuple(tokens[i * bs:(i + 1) * bs]))
            blk = table[i]
            have = self.children.get(key)
            if have is None:
                if blk in self.node_of:          # cached under another key: stop
                    break
                self.children[key] = blk
                self.node_of[blk] = key
                self.n_children[blk] = 0
                if parent is not None:
                    self.n_children[parent] += 1
            elif have != blk:
                break                            # the prefix is cached by other blocks
            self._tick(blk)
            parent = blk

    def append_slot(self, seq):
        """Reserve the next token slot of `seq`; returns (slot, cow_src, cow_dst)."""
        if seq in self.swapped:
            raise ValueError("sequence is swapped out")
        created = seq not in self.tables
        table = self.tables.setdefault(seq, [])
        pos = self.lens.get(seq, 0)
        bs = self.block_size
        cow = (-1, -1)
        if pos % bs == 0:
            try:
                table.append(self._pop())
            except OutOfBlocks:
                if created:                     # exhaustion changes nothing
                    del self.tables[seq]
                raise
        else:
            last = table[-1]
            if self.ref[last] > 1:
                new = self._pop()
                self.ref[last] -= 1
                table[-1] = new
                cow = (last, new)
        self.lens[seq] = pos + 1
        return table[-1] * bs + pos % bs, cow[0], cow[1]

    def fork(self, parent, child):
        if child in self.tables or child in self.swapped or parent not in self.tables:
            raise KeyError("fork needs an existing parent and a new child")
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]
        for blk in self.tables[child]:
            self.ref[blk] += 1

    def free(self, seq):
        if seq in self.swapped:
            self.swapped.discard(seq)
            del self.lens[seq]
            return
        for blk in self.tables.pop(seq):
            self._release(blk)
        del self.lens[seq]

    def swap_out(self, seq):
        """Release a resident sequence's blocks; returns them in logical order."""
        if seq not in self.tables:
            raise KeyError("swap_out needs a resident sequence")
        blocks = self.tables.pop(seq)
        for blk in blocks:
            self._release(blk)
        self.swapped.add(seq)
        return blocks

    def swap_in(self, seq):
        """Give a swapped sequence fresh blocks; returns them in logical order."""
        if seq not in self.swapped:
            raise KeyError("swap_in needs a swapped sequence")
        n = -(-self.lens[seq] // self.block_size)
        if len(self.free_pool) + len(self._evictable_chain()) < n:
            raise OutOfBlocks("not enough free blocks to swap in")
        blocks = [self._pop() for _ in range(n)]
        self.tables[seq] = blocks
        self.swapped.discard(seq)
        return blocks

    def _evictable_chain(self):
        """Blocks that repeated leaf evictions could free, in eviction order."""
        n_children = dict(self.n_children)
        out, cand = [], set(self._evictable())
        while cand:
            blk = min(cand, key=lambda b: self.stamp[b])
            cand.discard(blk)
            out.append(blk)
            parent = self.node_of[blk][0]
            if parent is not None:
                n_children[parent] -= 1
                if n_children[parent] == 0 and self.ref[parent] == 0:
                    cand.add(parent)
        return out

    def export_table(self, seqs, max_blocks, pad=0):
        rows = []
        for s in seqs:
            if s in self.swapped:
                raise ValueError("sequence is swapped out")
            t = self.tables.get(s, [])
            if len(t) > max_blocks:
                raise ValueError("table wider than max_blocks")
            rows.append(list(t) + [pad] * (max_blocks - len(t)))
        return rows
