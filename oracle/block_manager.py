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
  * prefix caching across requests (the pages: a server hashes block contents
    so that any two requests with a common prefix share the same physical
    blocks; llminference.xinbetween.com S06, "What's next"; the same page's
    "Production notes" on a radix tree of prefixes).  This model keys a cached
    block by its whole token prefix, the plain definition of "same content":
    the keys and values of a block depend on every token up to its end.
    Readings: only full blocks of an admitted prompt are cached and looked up;
    the lookup walks the prompt's full blocks from the first and stops at the
    first miss; at least the prompt's last token is always left to compute, so
    at most (n - 1) // B blocks are reused; a block whose count drops to zero
    stays cached and becomes evictable; new blocks come from the free list
    first and only then from the least recently retired evictable block; a
    retiring table's cached blocks become evictable deepest first (the tail
    goes before the shared prompt); evicting a block also drops every cached
    block whose prefix extends it (it can no longer be reached), and those go
    to the free list in ascending id order.
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
        self.prefix_cache = False
        self.index: dict[tuple, int] = {}        # token prefix -> cached block
        self.block_key: dict[int, tuple] = {}    # cached block -> its token prefix
        self.evictable: dict[int, int] = {}      # cached block with count 0 -> retire tick
        self.tick = 0
        self.prefix_query_tokens = 0
        self.prefix_hit_tokens = 0

    # -- allocation -------------------------------------------------------
    def _capacity(self) -> int:
        return len(self.free) + len(self.evictable)

    def _uncache(self, blk: int) -> None:
        del self.index[self.block_key.pop(blk)]
        self.evictable.pop(blk, None)

    def _take(self) -> int:
        """A block for a new table entry: the free list first, then the least
        recently retired evictable cached block."""
        if self.free:
            blk = self.free.pop()
        else:
            blk = min(self.evictable, key=self.evictable.get)
            key = self.block_key[blk]
            self._uncache(blk)
            below = sorted(b for k, b in self.index.items() if len(k) > len(key) and k[:len(key)] == key)
            for b in below:
                assert b in self.evictable, "a reachable-only-through-evicted block is in use"
                self._uncache(b)
                self.free.append(b)
        self.refcount[blk] = 1
        return blk

    def _release_device(self, table) -> None:
        for blk in table:
            self.refcount[blk] -= 1
            if self.refcount[blk] == 0 and blk not in self.block_key:
                self.free.append(blk)
        for blk in reversed(table):
            if self.refcount[blk] == 0 and blk in self.block_key and blk not in self.evictable:
                self.evictable[blk] = self.tick
                self.tick += 1

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
            dst = self._take()
            self.refcount[src] -= 1
            table[-1] = dst
            cow.append((src, dst))
            self.cow_copies += 1
        slots = []
        for t in range(length, length + n_new):
            if t % b == 0:
                table.append(self._take())
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
        if self._needs(seq, n_new, {}) > self._capacity():
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
        if need > self._capacity():
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
        self._release_device(self.tables.pop(seq, []))

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
    def _move(seqs, src_tables, dst_tables, release, dst_counts, take):
        """Copy the distinct blocks of the listed tables from one pool to the
        other, then retire the source tables.  Returns the (src, dst) pairs."""
        mapping: dict[int, int] = {}
        pairs = []
        for s in seqs:
            new = []
            for blk in src_tables[s]:
                if blk not in mapping:
                    mapping[blk] = take()
                    dst_counts[mapping[blk]] = 0
                    pairs.append((blk, mapping[blk]))
                dst_counts[mapping[blk]] += 1
                new.append(mapping[blk])
            dst_tables[s] = new
        for s in seqs:
            release(src_tables.pop(s))
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
        pairs = self._move(seqs, self.tables, self.host_tables, self._release_device,
                           self.host_refcount, self.host_free.pop)
        self.swap_out_blocks += len(pairs)
        return pairs

    def swap_in(self, seqs):
        """Move the listed swapped sequences back to device blocks; returns the
        (host block, device block) copies to run before the sequences are
        read.  All or nothing: OutOfBlocks when device blocks are short."""
        seqs = self._distinct(seqs, self.host_tables)
        need = len({blk for s in seqs for blk in self.host_tables[s]})
        if need > self._capacity():
            raise OutOfBlocks("not enough free device blocks")
        pairs = self._move(seqs, self.host_tables, self.tables,
                           lambda t: self._release(t, self.host_refcount, self.host_free),
                           self.refcount, self._take)
        self.swap_in_blocks += len(pairs)
        return pairs

    def is_swapped(self, seq: int) -> bool:
        if seq not in self.lengths:
            raise KeyError(seq)
        return seq in self.host_tables

    # -- prefix caching across requests ----------------------------------
    def enable_prefix_cache(self) -> None:
        if self.lengths:
            raise ValueError("enable the prefix cache before any sequence exists")
        self.prefix_cache = True

    def append_prompt(self, seq: int, tokens):
        """Admit a new sequence with its prompt token ids.  Leading full
        blocks whose token prefix is cached are shared instead of allocated;
        returns (slots, cached_tokens) with slot -1 for every cached token (its
        keys and values are already in the pool).  The prompt's new full blocks
        are cached once the call returns; their rows must be written (on the
        stream that later reads them) before another request can read them.
        All or nothing."""
        if not self.prefix_cache:
            raise ValueError("prefix cache is not enabled")
        if seq in self.lengths:
            raise ValueError(f"sequence {seq} exists")
        tokens = tuple(int(t) for t in tokens)
        n, b = len(tokens), self.block_size
        hits = []
        for j in range((n - 1) // b if n else 0):
            blk = self.index.get(tokens[:(j + 1) * b])
            if blk is None:
                break
            hits.append(blk)
        new = -(-n // b) - len(hits)
        revived = sum(1 for blk in hits if blk in self.evictable)
        if new > self._capacity() - revived:
            self.alloc_failures += 1
            raise OutOfBlocks(f"sequence {seq}: not enough free blocks")
        self.prefix_query_tokens += n
        self.prefix_hit_tokens += len(hits) * b
        for blk in hits:
            self.evictable.pop(blk, None)
            self.refcount[blk] += 1
        table = list(hits)
        while len(table) < -(-n // b):
            table.append(self._take())
        self.tables[seq] = table
        self.lengths[seq] = n
        for j in range(len(hits), n // b):
            key = tokens[:(j + 1) * b]
            if key not in self.index:
                self.index[key] = table[j]
                self.block_key[table[j]] = key
        cached = len(hits) * b
        slots = [-1] * cached + [table[t // b] * b + t % b for t in range(cached, n)]
        return slots, cached

    def is_cached(self, blk: int) -> bool:
        return blk in self.block_key

    # -- queries --------------------------------------------------------
    def table(self, seq: int) -> list[int]:
        """Device table of a resident sequence, host table of a swapped one."""
        if seq in self.host_tables:
            return list(self.host_tables[seq])
        return list(self.tables[seq])

    def length(self, seq: int) -> int:
        return self.lengths[seq]

    def stats(self) -> dict:
        used = self.num_blocks - len(self.free) - len(self.evictable)
        return dict(num_blocks=self.num_blocks, free_blocks=len(self.free),
                    used_blocks=used, num_seqs=len(self.lengths),
                    logical_tokens=sum(self.lengths.values()),
                    shared_blocks=sum(1 for c in self.refcount if c > 1),
                    alloc_failures=self.alloc_failures, cow_copies=self.cow_copies,
                    host_blocks=self.num_host_blocks, free_host_blocks=len(self.host_free),
                    swapped_seqs=len(self.host_tables), swap_out_blocks=self.swap_out_blocks,
                    swap_in_blocks=self.swap_in_blocks, cached_blocks=len(self.index),
                    evictable_blocks=len(self.evictable), prefix_query_tokens=self.prefix_query_tokens,
                    prefix_hit_tokens=self.prefix_hit_tokens)

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
            parked = set(self.evictable) if counts is self.refcount else set()
            assert not free & parked, "block both free and evictable"
            for blk in range(n):
                assert (blk in free or blk in parked) == (named[blk] == 0), f"block {blk} leaked or aliased"
        assert len(self.index) == len(self.block_key)
        for key, blk in self.index.items():
            assert self.block_key[blk] == key and len(key) % self.block_size == 0 and key
            assert (self.refcount[blk] == 0) == (blk in self.evictable), f"cached block {blk} count/evictable"
            if len(key) > self.block_size:
                assert key[:-self.block_size] in self.index, f"cached block {blk} has no cached parent"
