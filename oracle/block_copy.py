"""Oracle of the copy-on-write block copy.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources:

* "大模型推理引擎优化：KV Cache 与连续批处理" (devpress.csdn.net), §4.2: sequences may share
  KV-cache blocks; before one of them writes into a shared block it must get its
  own copy (copy-on-write), which the block manager tracks with reference counts.
* "LLM推理引擎深度实战：从PagedAttention到分布式推理部署", §2.2: copy-on-write lets beam
  search and parallel sampling share the blocks of a common prefix until a
  sequence changes one.  §3.2: a preempted request's pages are written out to
  CPU memory and read back to the GPU when it resumes (swap-out / swap-in).

Swap (the same reading across two pools): for every pair (src, dst), block src
of the source pools becomes block dst of the destination pools, K, V and FP8
scales alike; pairs outside either pool change nothing.

What is copied by the copy-on-write step (the plainest reading): for every pair (src, dst) the whole
physical block src of the K pool and of the V pool, and for an FP8 cache the
block's 16 per-token scales of each, become block dst's contents.  Pairs with
src or dst outside [0, num_blocks), or src == dst, change nothing.  All pairs
read the pools as they were before the call (the destinations of one call are
distinct and are not sources in the same call).
"""

import numpy as np


def copy_blocks(key_cache, value_cache, block_mapping, k_scale=None, v_scale=None):
    """New (key_cache, value_cache, k_scale, v_scale) after the copies of block_mapping [n, 2].

    Pools are arrays shaped [num_blocks, 16, Hkv, D] (any dtype: bit patterns are moved
    unchanged); scales [num_blocks, 16] float32 or None.
    """
    before = [key_cache, value_cache, k_scale, v_scale]
    after = [None if a is None else np.array(a, copy=True) for a in before]
    num_blocks = key_cache.shape[0]
    for src, dst in np.asarray(block_mapping, dtype=np.int64).reshape(-1, 2):
        if not (0 <= src < num_blocks and 0 <= dst < num_blocks) or src == dst:
            continue
        for old, new in zip(before, after):
            if old is not None:
                new[dst] = old[src]
    return tuple(after)


def swap_blocks(src, dst, block_mapping):
    """New destination pools after copying block src of ``src`` to block dst of ``dst``.

    src, dst: tuples (key_cache, value_cache, k_scale, v_scale) of arrays (scales may be
    None); block_mapping [n, 2] int (src, dst) pairs.  Arguments are not modified.
    """
    out = [None if a is None else np.array(a, copy=True) for a in dst]
    n_src, n_dst = src[0].shape[0], dst[0].shape[0]
    for s, d in np.asarray(block_mapping, dtype=np.int64).reshape(-1, 2):
        if not (0 <= s < n_src and 0 <= d < n_dst):
            continue
        for a, b in zip(src, out):
            if a is not None:
                b[d] = a[s]
    return tuple(out)
