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

    def _pop(self):
        if not self.free_pool:
            raise OutOfBlocks("KV block pool exhausted; preempt a sequence")
        blk = self.free_pool.pop()
        self.ref[blk] += 1
        return blk

    def append_slot(self, seq):
        """Reserve the next token slot of `seq`; returns (slot, cow_src, cow_dst)."""
        if seq in self.swapped:
            raise ValueError("sequence is swapped out")
        table = self.tables.setdefault(seq, [])
        pos = self.lens.get(seq, 0)
        bs = self.block_size
        cow = (-1, -1)
        if pos % bs == 0:
            table.append(self._pop())
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
            self.ref[blk] -= 1
            if self.ref[blk] == 0:
                self.free_pool.append(blk)
        del self.lens[seq]

    def swap_out(self, seq):
        """Release a resident sequence's blocks; returns them in logical order."""
        if seq not in self.tables:
            raise KeyError("swap_out needs a resident sequence")
        blocks = self.tables.pop(seq)
        for blk in blocks:
            self.ref[blk] -= 1
            if self.ref[blk] == 0:
                self.free_pool.append(blk)
        self.swapped.add(seq)
        return blocks

    def swap_in(self, seq):
        """Give a swapped sequence fresh blocks; returns them in logical order."""
        if seq not in self.swapped:
            raise KeyError("swap_in needs a swapped sequence")
        n = -(-self.lens[seq] // self.block_size)
        if len(self.free_pool) < n:
            raise OutOfBlocks("not enough free blocks to swap in")
        blocks = [self._pop() for _ in range(n)]
        self.tables[seq] = blocks
        self.swapped.discard(seq)
        return blocks

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
