"""Host-side block bookkeeping used to build page tables for the synthetic workloads.

Harness code only: it decides which physical block holds which logical block and holds
none of the attention arithmetic.  What it models, from the prose of "大模型推理引擎优化：KV
Cache 与连续批处理" (devpress.csdn.net, §2.2) and "LLM推理引擎深度实战：从PagedAttention到分布式
推理部署" (ybb.press, §2.2): the cache is cut into fixed 16-token blocks; a sequence gets
blocks only for tokens it holds (ceil(n / 16) for n tokens), anywhere in the pool; a block
that several sequences share (a common prefix) carries a count of its holders and returns
to the pool when the last one lets go; asking for more blocks than are free is an error.

The form is this module's own: the ids are handed out in one fixed order given up front
(the seeded permutation of the workloads), a cursor marks how far that order has been
used, blocks that come back wait in a queue that is drawn from once the order is used
up, and the holder counts live in one integer array indexed by block id.
"""

import numpy as np

BLOCK_SIZE = 16


def blocks_for(num_tokens):
    """Number of 16-token blocks needed to hold ``num_tokens`` tokens."""
    return -(-int(num_tokens) // BLOCK_SIZE)


def slot_of(block_ids, position):
    """Slot id (physical_block * 16 + offset) of logical token ``position``."""
    return int(block_ids[position // BLOCK_SIZE]) * BLOCK_SIZE + position % BLOCK_SIZE


class PoolExhausted(RuntimeError):
    pass


class BlockPool:
    """Physical block ids handed out in a fixed order, with a holder count per id."""

    def __init__(self, order):
        self._order = np.asarray(order, dtype=np.int64).reshape(-1)
        if self._order.size and (self._order.min() < 0 or np.unique(self._order).size != self._order.size):
            raise ValueError("block ids must be distinct and non-negative")
        self._cursor = 0                       # ids _order[_cursor:] were never handed out
        self._returned = []                    # ids given back, oldest first
        size = int(self._order.max()) + 1 if self._order.size else 0
        self._holders = np.zeros(size, dtype=np.int32)
        self.total = int(self._order.size)

    def num_free(self):
        return self.total - self._cursor + len(self._returned)

    def free_ids(self):
        """The free ids in the order the next allocations will take them."""
        return [int(b) for b in self._order[self._cursor:]] + list(self._returned)

    def allocate(self, num_blocks):
        num_blocks = int(num_blocks)
        if num_blocks > self.num_free():
            raise PoolExhausted(f"need {num_blocks} blocks, {self.num_free()} free")
        fresh = min(num_blocks, self.total - self._cursor)
        ids = [int(b) for b in self._order[self._cursor:self._cursor + fresh]]
        self._cursor += fresh
        ids += self._returned[:num_blocks - fresh]
        del self._returned[:num_blocks - fresh]
        self._holders[ids] = 1
        return ids

    def allocate_tokens(self, num_tokens):
        return self.allocate(blocks_for(num_tokens))

    def _held(self, b):
        return 0 <= b < self._holders.size and self._holders[b] > 0

    def share(self, blocks):
        """One more holder for each of ``blocks`` (all must be held already)."""
        blocks = [int(b) for b in blocks]
        if not all(self._held(b) for b in blocks):
            raise ValueError(f"sharing a block that is not allocated: {blocks}")
        for b in blocks:
            self._holders[b] += 1
        return blocks

    def release(self, blocks):
        """One holder less for each of ``blocks``; a block whose count reaches 0 is free again."""
        for b in (int(x) for x in blocks):
            if not self._held(b):
                raise ValueError(f"block {b} is not allocated")
            self._holders[b] -= 1
            if self._holders[b] == 0:
                self._returned.append(b)

    def utilization(self):
        """Share of the pool's blocks that some sequence holds."""
        return (self.total - self.num_free()) / self.total if self.total else 0.0
