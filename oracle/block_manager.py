"""Reference block manager: paging, sharing and copy-on-write, in plain Python.

What it models, and where the pages state it:
  * "KV Cache memory optimisation: from PagedAttention to AI memory systems"
    [P2] 2.2-2.3: the cache is cut into fixed blocks handed out on demand
    from a common pool, and returned to it when a request ends;
  * [P2] 3.1-3.2 and "The KV Cache memory ledger" [P5] 4: requests with the
    same prefix point at the same physical blocks; every block counts the
    sequences that reference it and goes back to the pool at zero; before a
    sequence writes into a block that others still reference, the block is
    copied and the write goes to the private copy ([P2] 7.2: doing this
    wrong corrupts the other sequences).

Behaviour (the native manager in the library must match it exactly):
  * the free list is a stack: blocks are taken from its end; `free_order`
    (default 0, 1, 2, ...) lists the order in which fresh blocks are taken;
    freed blocks are pushed back and reused first;
  * fork(parent, child): the child references every block of the parent,
    its last (possibly partial) block included, and has the same length;
  * append_slots(seqs): for each sequence in order, its next token goes to
    offset n % bs of its last block; a new block is taken when n % bs == 0;
    if that last block is partial and shared, a fresh block is taken, the
    pair (old, new) is recorded for copying, the old block loses one
    reference and the new one replaces it in the table; the call fails with
    nothing changed if the pool cannot supply every block it needs;
  * free(seq): every block loses one reference; blocks at zero are pushed
    back in table order.

Test infrastructure only (see the package docstring).
"""

from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple


class PoolExhausted(RuntimeError):
    pass


class ReferenceBlockManager:
    def __init__(self, num_blocks: int, block_size: int = 16,
                 free_order: Optional[Sequence[int]] = None):
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("free_order must be a permutation of the block ids")
        self.bs = block_size
        self.free: List[int] = order[::-1]            # the end of the list is taken first
        self.ref = [0] * num_blocks
        self.tables: Dict[int, List[int]] = {}
        self.lens: Dict[int, int] = {}

    def add_sequence(self, seq: int) -> None:
        if seq in self.tables:
            raise KeyError(seq)
        self.tables[seq] = []
        self.lens[seq] = 0

    def fork(self, parent: int, child: int) -> None:
        if child in self.tables or parent not in self.tables:
            raise KeyError(child)
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]
        for b in self.tables[child]:
            self.ref[b] += 1

    def append_slots(self, seqs: Sequence[int]) -> Tuple[List[int], List[Tuple[int, int]]]:
        for s in seqs:
            if s not in self.tables:
                raise KeyError(s)
        if len(set(seqs)) != len(seqs):
            raise ValueError("a sequence may appear once per call")
        need = 0
        for s in seqs:
            n, t = self.lens[s], self.tables[s]
            if n % self.bs == 0 or self.ref[t[-1]] > 1:
                need += 1
        if need > len(self.free):
            raise PoolExhausted("not enough free blocks")
        slots, copies = [], []
        for s in seqs:
            n, t = self.lens[s], self.tables[s]
            off = n % self.bs
            if off == 0:
                b = self.free.pop()
                self.ref[b] = 1
                t.append(b)
            elif self.ref[t[-1]] > 1:
                b = self.free.pop()
                self.ref[b] = 1
                copies.append((t[-1], b))
                self.ref[t[-1]] -= 1
                t[-1] = b
            slots.append(t[-1] * self.bs + off)
            self.lens[s] = n + 1
        return slots, copies

    def free_sequence(self, seq: int) -> None:
        for b in self.tables.pop(seq):
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)
        del self.lens[seq]

    def num_free(self) -> int:
        return len(self.free)
