"""Python model of the host block manager (free list, tables, refcounts, CoW).

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import or call anything in oracle/.  It is
the differential model for the C++ block manager of the product library.

Behaviour, each point from the pages:
  * one global free list of physical blocks; "ANY free block will do"
    (llminference.xinbetween.com S06 "PagedAttention", the BlockManager
    listing under "The solution"); blocks are taken from the end of the list
    and returned to it, so the most recently freed block is reused first;
  * a sequence starts with no block and takes one more whenever its length is
    a multiple of B before a write (mercemay.com "Paged KV Cache Allocation
    and the Block Table", the append_token listing under "Blocks, tables, and
    the indirection"; aicassindra.com "tm_paged_attention_deep", "Anatomy of
    a KV block");
  * the slot of logical position t is table[t // B] * B + t % B
    (synapticradio.com "The KV Cache Is an Allocator Problem", the equation in
    "What the trace shows");
  * every physical block carries a count of the tables naming it; forking a
    sequence aliases its table and increments those counts; retiring a
    sequence decrements the count of every block in its table and returns only
    those reaching zero (mercemay.com, "Sharing blocks between sequences");
  * a write into a block whose count exceeds one first copies that block to a
    fresh one, points the writer's table at the copy and decrements the
    original's count (copy-on-write at block granularity; aicassindra.com,
    "Copy-on-write for shared prefixes");
  * after every operation each block's count equals the number of tables
    naming it (S06 "PagedAttention", "Reference counts must be exact").

Readings where the pages leave a choice open:
  * the listing grows a table block by block and returns False when the list
    runs dry, leaving a partial append behind; here an append that cannot be
    satisfied changes nothing and raises OutOfBlocks;
  * the copy is taken only when the written block is shared, so the last
    holder writes in place: n forks of a prefix whose last block is partial
    make n - 1 copies;
  * freeing an unknown sequence is a no-op, as the listing's
    tables.pop(req_id, []) is;
  * the initial free-list order is a parameter: the first block handed out is
    initial_order[0]; by default blocks leave in ascending order, as the
    simulator's block tables show (S06, "Try it").
"""
from __future__ import annotations


class OutOfBlocks(RuntimeError):
    pass


class BlockManagerModel:
    def __init__(self, num_blocks: int, block_size: int, initial_order=None):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("sizes must be positive")
        order = list(range(num_blocks)) if initial_order is None else [int(b) for b in initial_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("initial order must be a permutation of the pool")
        self.num_blocks = num_blocks
        self.block_size = block_size
        # End of the list is taken first, so store the order reversed.
        self.free = order[::-1]
        self.refcount = [0] * num_blocks
        self.tables: dict[int, list[int]] = {}
        self.lengths: dict[int, int] = {}
        self.alloc_failures = 0
        self.cow_copies = 0

    # -- sizing ---------------------------------------------------------
    def _needs(self, seq: int, n_new: int, refcount_delta: dict) -> int:
        """Free blocks consumed by appending n_new tokens to seq."""
        length = self.lengths.get(seq, 0)
        table = self.tables.get(seq, [])
        b = self.block_size
        need = -(-(length + n_new) // b) - len(table)
        if n_new > 0 and length % b != 0:
            last = table[-1]
            if self.refcount[last] + refcount_delta.get(last, 0) > 1:
                need += 1
                refcount_delta[last] = refcount_delta.get(last, 0) - 1
        return need

    # -- operations -----------------------------------------------------
    def _append_unchecked(self, seq: int, n_new: int):
        b = self.block_size
        table = self.tables.setdefault(seq, [])
        length = self.lengths.setdefault(seq, 0)
        cow = []
        if n_new > 0 and length % b != 0 and self.refcount[table[-1]] > 1:
            src = table[-1]
            dst = self.free.pop()
            self.refcount[src] -= 1
            self.refcount[dst] = 1
            table[-1] = dst
            cow.append((src, dst))
            self.cow_copies += 1
        slots = []
        for t in range(length, length + n_new):
            if t % b == 0:
                blk = self.free.pop()
                self.refcount[blk] = 1
                table.append(blk)
            slots.append(table[t // b] * b + t % b)
        self.lengths[seq] = length + n_new
        return slots, cow

    def append(self, seq: int, n_new: int = 1):
        """Append n_new tokens; returns (slots, cow_pairs).  All or nothing."""
        if n_new < 0:
            raise ValueError("n_new must be >= 0")
        if self._needs(seq, n_new, {}) > len(self.free):
            self.alloc_failures += 1
            raise OutOfBlocks(f"sequence {seq}: not enough free blocks")
        return self._append_unchecked(seq, n_new)

    def append_step(self, seqs):
        """One token for each listed (distinct) sequence, in order; all or nothing."""
        seqs = [int(s) for s in seqs]
        if len(set(seqs)) != len(seqs):
            raise ValueError("a sequence may appear once per step")
        delta: dict = {}
        need = sum(self._needs(s, 1, delta) for s in seqs)
        if need > len(self.free):
            self.alloc_failures += 1
            raise OutOfBlocks("step does not fit in the free list")
        slots, cows = [], []
        for s in seqs:
            sl, cw = self._append_unchecked(s, 1)
            slots.extend(sl)
            cows.extend(cw)
        return slots, cows

    def fork(self, parent: int, child: int) -> None:
        if parent not in self.tables:
            raise KeyError(parent)
        if child in self.tables:
            raise ValueError(f"sequence {child} exists")
        self.tables[child] = list(self.tables[parent])
        self.lengths[child] = self.lengths[parent]
        for blk in self.tables[child]:
            self.refcount[blk] += 1

    def free_seq(self, seq: int) -> None:
        table = self.tables.pop(seq, [])
        self.lengths.pop(seq, None)
        for blk in table:
            self.refcount[blk] -= 1
            if self.refcount[blk] == 0:
                self.free.append(blk)

    # -- queries --------------------------------------------------------
    def table(self, seq: int) -> list[int]:
        return list(self.tables[seq])

    def length(self, seq: int) -> int:
        return self.lengths[seq]

    def stats(self) -> dict:
        used = self.num_blocks - len(self.free)
        return dict(num_blocks=self.num_blocks, free_blocks=len(self.free),
                    used_blocks=used, num_seqs=len(self.tables),
                    logical_tokens=sum(self.lengths.values()),
                    shared_blocks=sum(1 for c in self.refcount if c > 1),
                    alloc_failures=self.alloc_failures, cow_copies=self.cow_copies)

    def check(self) -> None:
        """Raise AssertionError unless counts equal table references exactly."""
        named = [0] * self.num_blocks
        for seq, table in self.tables.items():
            assert len(table) == -(-self.lengths[seq] // self.block_size), seq
            for blk in table:
                named[blk] += 1
        assert named == self.refcount, "refcount differs from table references"
        free = set(self.free)
        assert len(free) == len(self.free), "block listed twice as free"
        for blk in range(self.num_blocks):
            assert (blk in free) == (named[blk] == 0), f"block {blk} leaked or aliased"
