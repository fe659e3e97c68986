"""Plain model of the paged block manager.

TEST INFRASTRUCTURE ONLY: the tests compare the library's host block
manager (pa_bm_*) with this model operation by operation; nothing in the
product path imports it, and it imports nothing from the product package.

What it models ("PagedAttention: The Cache Was Storing Nothing"):
  §2.2 "Borrowing paging from the 1960s": the cache is cut into fixed-size
  blocks, each request has a block table from logical to physical blocks,
  any free block will do (all have the same size), and only a request's
  last block is partly filled;
  §2.3 "What the table buys that reservations could not": tables may point
  at the same physical blocks, and a block is copied only when a sequence
  diverges and writes into it.
The id policy is the library's own (the pages fix none): never-used
blocks in id order first (a bump pointer), released blocks reused most
recent first (a LIFO free list).  The model keeps it in the plainest form:
a counter, a Python list used as a stack, and a dict of reference counts.
"""
from __future__ import annotations

OK, ERR_NULL, ERR_SHAPE, ERR_TABLE, ERR_NOMEM = 0, 1, 2, 8, 10


class BlockManagerModel:
    def __init__(self, num_blocks: int, block_size: int):
        assert num_blocks > 0 and block_size > 0
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.next_unused = 0      # blocks next_unused .. num_blocks-1 never handed out
        self.released = []        # stack of released blocks, top = most recent
        self.refs = {}            # block -> number of table entries pointing at it

    def num_free(self) -> int:
        return (self.num_blocks - self.next_unused) + len(self.released)

    def refcount(self, block: int) -> int:
        if not 0 <= block < self.num_blocks:
            return -1
        return self.refs.get(block, 0)

    def _take(self) -> int:
        if self.released:
            block = self.released.pop()
        elif self.next_unused < self.num_blocks:
            block = self.next_unused
            self.next_unused += 1
        else:
            return -1
        self.refs[block] = 1
        return block

    def alloc(self, n: int):
        if n < 0:
            return ERR_SHAPE, []
        if self.num_free() < n:
            return ERR_NOMEM, []
        return OK, [self._take() for _ in range(n)]

    def release(self, ids) -> int:
        for block in ids:
            if self.refcount(block) <= 0:
                return ERR_TABLE
            self.refs[block] -= 1
            if self.refs[block] == 0:
                del self.refs[block]
                self.released.append(block)
        return OK

    def share(self, ids) -> int:
        for block in ids:
            if self.refcount(block) <= 0:
                return ERR_TABLE
            self.refs[block] += 1
        return OK

    def prepare_append(self, tables, seq_lens):
        """tables: list of lists (rows of equal length), updated in place.
        Returns (status, positions, cow pairs).  All or nothing: the step is
        first checked on a copy of the state, then applied."""
        B = self.block_size
        positions = [-1] * len(seq_lens)
        # dry run on copies: errors leave everything as it was
        saved = (self.next_unused, list(self.released), dict(self.refs))
        rows = [list(r) for r in tables]
        status = self._append_step(rows, seq_lens, positions, [])
        self.next_unused, self.released, self.refs = saved
        if status != OK:
            return status, [-1] * len(seq_lens), []
        cows = []
        self._append_step(tables, seq_lens, positions, cows)
        return OK, positions, cows

    def _append_step(self, tables, seq_lens, positions, cows):
        B = self.block_size
        for b, L in enumerate(seq_lens):
            if L < 0:
                continue
            j = L // B
            if j >= len(tables[b]):
                return ERR_TABLE
            if L % B == 0:  # the new token opens a block
                block = self._take()
                if block < 0:
                    return ERR_NOMEM
                tables[b][j] = block
            else:           # it lands in the current last block
                old = tables[b][j]
                if self.refcount(old) <= 0:
                    return ERR_TABLE
                if self.refs[old] > 1:  # shared: copy before writing
                    block = self._take()
                    if block < 0:
                        return ERR_NOMEM
                    cows.append((old, block))
                    self.release([old])
                    tables[b][j] = block
            positions[b] = L
        return OK
