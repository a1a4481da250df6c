"""Host-side block bookkeeping used to build page tables for the synthetic workloads.

This is harness code: it decides which physical block holds which logical
block, the way the block manager of "大模型推理引擎优化：KV Cache 与连续批处理"
(devpress.csdn.net, §2.2 and §三) does: fixed 16-token blocks, handed out from
the front of a free list on demand (a request for n tokens takes ceil(n/16)
blocks), an error when the pool runs short, reference counts for blocks that
several sequences share (prefix sharing, "LLM推理引擎深度实战：从PagedAttention到分布式推理
部署" §2.2), and a block going back to the end of the free list once its last
holder releases it.  It holds none of the attention arithmetic.
"""

from collections import deque

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
    """FIFO free list of physical block ids with per-block reference counts."""

    def __init__(self, order):
        self.free = deque(int(b) for b in order)
        self.total = len(self.free)
        self.refs = {}

    def allocate(self, num_blocks):
        if num_blocks > len(self.free):
            raise PoolExhausted(f"need {num_blocks} blocks, {len(self.free)} free")
        out = [self.free.popleft() for _ in range(num_blocks)]
        for b in out:
            self.refs[b] = 1
        return out

    def allocate_tokens(self, num_tokens):
        return self.allocate(blocks_for(num_tokens))

    def share(self, blocks):
        for b in blocks:
            if self.refs.get(b, 0) <= 0:
                raise ValueError(f"block {b} is not allocated")
            self.refs[b] += 1
        return list(blocks)

    def release(self, blocks):
        for b in blocks:
            n = self.refs.get(b, 0)
            if n <= 0:
                raise ValueError(f"block {b} is not allocated")
            if n == 1:
                del self.refs[b]
                self.free.append(b)
            else:
                self.refs[b] = n - 1

    def utilization(self):
        return (self.total - len(self.free)) / self.total if self.total else 0.0
