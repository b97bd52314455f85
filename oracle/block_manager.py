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
    naming it (S06 "PagedAttention", "Reference counts must be exact");
  * when blocks run out, a sequence's blocks can be copied out to host memory
    and back later instead of recomputing it (mercemay.com, "Three ways
    contiguous reservation loses memory" and the closing paragraphs of
    "Blocks, tables, and the indirection"; llminference.xinbetween.com S06,
    the third exercise: drive the allocator to exhaustion, then swap or
    recompute).

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
    simulator's block tables show (S06, "Try it");
  * swapping (the pages name the option, not its bookkeeping): host memory is
    a second pool of blocks with its own free list and counts, run with the
    device list's discipline (ascending at first, last retired reused first).
    Swapping out a set of sequences copies every distinct device block of
    their tables once, in table order, so sequences that shared a block share
    its host copy; then each table is retired as free_seq retires it.  A
    block that a resident sequence still names stays on the device and is
    copied as well.  Swapping in is the mirror image.  A swapped sequence
    keeps its length, cannot grow or fork, and free_seq releases its host
    blocks.  Both directions are all or nothing.
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
        self.num_host_blocks = 0
        self.host_free: list[int] = []
        self.host_refcount: list[int] = []
        self.host_tables: dict[int, list[int]] = {}
        self.swap_out_blocks = 0
        self.swap_in_blocks = 0

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

    def _resident(self, seq: int) -> None:
        if seq in self.host_tables:
            raise ValueError(f"sequence {seq} is swapped out")

    def append(self, seq: int, n_new: int = 1):
        """Append n_new tokens; returns (slots, cow_pairs).  All or nothing."""
        if n_new < 0:
            raise ValueError("n_new must be >= 0")
        self._resident(seq)
        if self._needs(seq, n_new, {}) > len(self.free):
            self.alloc_failures += 1
            raise OutOfBlocks(f"sequence {seq}: not enough free blocks")
        return self._append_unchecked(seq, n_new)

    def append_step(self, seqs):
        """One token for each listed (distinct) sequence, in order; all or nothing."""
        seqs = [int(s) for s in seqs]
        if len(set(seqs)) != len(seqs):
            raise ValueError("a sequence may appear once per step")
        for s in seqs:
            self._resident(s)
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
        self._resident(parent)
        if parent not in self.tables:
            raise KeyError(parent)
        if child in self.lengths:
            raise ValueError(f"sequence {child} exists")
        self.tables[child] = list(self.tables[parent])
        self.lengths[child] = self.lengths[parent]
        for blk in self.tables[child]:
            self.refcount[blk] += 1

    def free_seq(self, seq: int) -> None:
        self.lengths.pop(seq, None)
        if seq in self.host_tables:
            self._release(self.host_tables.pop(seq), self.host_refcount, self.host_free)
            return
        self._release(self.tables.pop(seq, []), self.refcount, self.free)

    @staticmethod
    def _release(table, counts, free) -> None:
        for blk in table:
            counts[blk] -= 1
            if counts[blk] == 0:
                free.append(blk)

    # -- swapping to host memory -----------------------------------------
    def set_host_blocks(self, n: int) -> None:
        """Size the host swap pool (allowed while nothing is swapped out)."""
        if n < 0:
            raise ValueError("host block count must be >= 0")
        if self.host_tables:
            raise ValueError("sequences are swapped out")
        self.num_host_blocks = n
        self.host_free = list(range(n))[::-1]
        self.host_refcount = [0] * n

    @staticmethod
    def _move(seqs, src_tables, dst_tables, src_counts, src_free, dst_counts, dst_free):
        """Copy the distinct blocks of the listed tables from one pool to the
        other, then retire the source tables.  Returns the (src, dst) pairs."""
        mapping: dict[int, int] = {}
        pairs = []
        for s in seqs:
            new = []
            for blk in src_tables[s]:
                if blk not in mapping:
                    mapping[blk] = dst_free.pop()
                    pairs.append((blk, mapping[blk]))
                dst_counts[mapping[blk]] += 1
                new.append(mapping[blk])
            dst_tables[s] = new
        for s in seqs:
            BlockManagerModel._release(src_tables.pop(s), src_counts, src_free)
        return pairs

    def _distinct(self, seqs, tables) -> list[int]:
        seqs = [int(s) for s in seqs]
        if len(set(seqs)) != len(seqs):
            raise ValueError("a sequence may appear once per call")
        for s in seqs:
            if s not in tables:
                raise KeyError(s)
        return seqs

    def swap_out(self, seqs):
        """Move the listed resident sequences to host blocks; returns the
        (device block, host block) copies to run before the device blocks are
        reused.  All or nothing: OutOfBlocks when host blocks are short."""
        seqs = self._distinct(seqs, self.tables)
        need = len({blk for s in seqs for blk in self.tables[s]})
        if need > len(self.host_free):
            raise OutOfBlocks("not enough free host blocks")
        pairs = self._move(seqs, self.tables, self.host_tables, self.refcount, self.free,
                           self.host_refcount, self.host_free)
        self.swap_out_blocks += len(pairs)
        return pairs

    def swap_in(self, seqs):
        """Move the listed swapped sequences back to device blocks; returns the
        (host block, device block) copies to run before the sequences are
        read.  All or nothing: OutOfBlocks when device blocks are short."""
        seqs = self._distinct(seqs, self.host_tables)
        need = len({blk for s in seqs for blk in self.host_tables[s]})
        if need > len(self.free):
            raise OutOfBlocks("not enough free device blocks")
        pairs = self._move(seqs, self.host_tables, self.tables, self.host_refcount, self.host_free,
                           self.refcount, self.free)
        self.swap_in_blocks += len(pairs)
        return pairs

    def is_swapped(self, seq: int) -> bool:
        if seq not in self.lengths:
            raise KeyError(seq)
        return seq in self.host_tables

    # -- queries --------------------------------------------------------
    def table(self, seq: int) -> list[int]:
        """Device table of a resident sequence, host table of a swapped one."""
        if seq in self.host_tables:
            return list(self.host_tables[seq])
        return list(self.tables[seq])

    def length(self, seq: int) -> int:
        return self.lengths[seq]

    def stats(self) -> dict:
        used = self.num_blocks - len(self.free)
        return dict(num_blocks=self.num_blocks, free_blocks=len(self.free),
                    used_blocks=used, num_seqs=len(self.lengths),
                    logical_tokens=sum(self.lengths.values()),
                    shared_blocks=sum(1 for c in self.refcount if c > 1),
                    alloc_failures=self.alloc_failures, cow_copies=self.cow_copies,
                    host_blocks=self.num_host_blocks, free_host_blocks=len(self.host_free),
                    swapped_seqs=len(self.host_tables), swap_out_blocks=self.swap_out_blocks,
                    swap_in_blocks=self.swap_in_blocks)

    def check(self) -> None:
        """Raise AssertionError unless counts equal table references exactly."""
        assert not set(self.tables) & set(self.host_tables), "sequence both resident and swapped"
        assert set(self.tables) | set(self.host_tables) == set(self.lengths), "length without a table"
        for tables, counts, free_list, n in ((self.tables, self.refcount, self.free, self.num_blocks),
                                             (self.host_tables, self.host_refcount, self.host_free,
                                              self.num_host_blocks)):
            named = [0] * n
            for seq, table in tables.items():
                assert len(table) == -(-self.lengths[seq] // self.block_size), seq
                for blk in table:
                    named[blk] += 1
            assert named == counts, "refcount differs from table references"
            free = set(free_list)
            assert len(free) == len(free_list), "block listed twice as free"
            for blk in range(n):
                assert (blk in free) == (named[blk] == 0), f"block {blk} leaked or aliased"
