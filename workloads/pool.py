"""Host-side physical block pool used to build block tables.

Blocks are handed out on demand from a free list (any free block will do, so
the list is a seeded permutation), every block carries a reference count, a
fork lets a second sequence point at the same physical blocks, and a block
returns to the free list when its count drops to zero.  This follows the
block-manager behaviour described on "Large-model inference KV Cache memory
optimisation: from PagedAttention to AI memory systems" (wmrh.cn), sections
2.2-2.3 (on-demand allocation, recycling) and 3.1-3.2 (sharing, reference
counts), and "The KV Cache memory ledger" (gcssc.sfwss.com), section 4.

It is support code for building inputs; it never runs on the device.
"""

from __future__ import annotations

from typing import Dict, Iterable, List


class PoolExhausted(RuntimeError):
    pass


class BlockPool:
    def __init__(self, num_blocks: int, free_order: Iterable[int], block_size: int = 16):
        order = [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("free_order must be a permutation of range(num_blocks)")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self._free: List[int] = order[::-1]          # pop() takes from the front of `order`
        self.refcount = [0] * num_blocks
        self.tables: Dict[int, List[int]] = {}
        self.num_tokens: Dict[int, int] = {}

    # -- blocks -----------------------------------------------------------
    def allocate(self) -> int:
        if not self._free:
            raise PoolExhausted("no free physical block")
        b = self._free.pop()
        assert self.refcount[b] == 0
        self.refcount[b] = 1
        return b

    def release(self, b: int) -> None:
        if self.refcount[b] <= 0:
            raise ValueError(f"block {b} released more times than referenced")
        self.refcount[b] -= 1
        if self.refcount[b] == 0:
            self._free.append(b)

    @property
    def num_free(self) -> int:
        return len(self._free)

    # -- sequences --------------------------------------------------------
    def new_sequence(self, seq: int) -> None:
        if seq in self.tables:
            raise ValueError(f"sequence {seq} exists")
        self.tables[seq] = []
        self.num_tokens[seq] = 0

    def append_token(self, seq: int) -> int:
        """Reserve room for one more token of `seq`; return its flat slot.

        A new block is taken only when the sequence's last block is full.
        The flat slot is physical_block * block_size + offset_in_block.
        """
        n = self.num_tokens[seq]
        table = self.tables[seq]
        off = n % self.block_size
        if off == 0:
            table.append(self.allocate())
        elif self.refcount[table[-1]] > 1:
            raise NotImplementedError("append into a shared partial block needs copy-on-write")
        self.num_tokens[seq] = n + 1
        return table[-1] * self.block_size + off

    def fork(self, parent: int, child: int, num_tokens: int) -> None:
        """Child starts with the parent's first `num_tokens` tokens, shared.

        Only whole blocks are shared, so `num_tokens` must be a multiple of
        the block size.
        """
        if num_tokens % self.block_size:
            raise ValueError("only whole blocks can be shared")
        nb = num_tokens // self.block_size
        src = self.tables[parent][:nb]
        if len(src) != nb:
            raise ValueError("parent is shorter than the shared prefix")
        self.new_sequence(child)
        for b in src:
            self.refcount[b] += 1
        self.tables[child] = list(src)
        self.num_tokens[child] = num_tokens

    def free_sequence(self, seq: int) -> None:
        for b in self.tables.pop(seq):
            self.release(b)
        del self.num_tokens[seq]
