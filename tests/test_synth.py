"""Host logic: the block pool that builds page tables, and the synthetic workloads' invariants."""

import numpy as np
import pytest
import torch

import synth
from synth import BlockPool, PoolExhausted, blocks_for, slot_of, bits_np


def test_blocks_for_is_ceiling_of_tokens_over_16():
    assert [blocks_for(n) for n in (0, 1, 15, 16, 17, 32, 33)] == [0, 1, 1, 1, 2, 2, 3]


def test_pool_order_exhaustion_and_refcounts():
    pool = BlockPool([5, 3, 9, 1])
    a = pool.allocate_tokens(17)          # ceil(17 / 16) = 2 blocks, in the given order
    assert a == [5, 3]
    with pytest.raises(PoolExhausted):
        pool.allocate(3)
    assert pool.free_ids() == [9, 1]       # a failed request takes nothing
    pool.share(a)                          # a second holder
    pool.release(a)
    assert pool.free_ids() == [9, 1]       # still held once
    assert pool.utilization() == 0.5
    pool.release(a)
    assert pool.free_ids() == [9, 1, 5, 3]  # given back after the never-used ids, in order
    assert pool.utilization() == 0.0
    with pytest.raises(ValueError):
        pool.release([5])
    with pytest.raises(ValueError):
        pool.share([9])
    assert pool.allocate(3) == [9, 1, 5]    # never-used ids first, then returned ones
    assert pool.allocate_tokens(0) == []


def test_slot_of():
    assert slot_of([7, 2], 0) == 112 and slot_of([7, 2], 15) == 127 and slot_of([7, 2], 16) == 32


@pytest.mark.parametrize("name", ["tiny", "gqa70b", "fp8beams"])
def test_workload_invariants(name):
    w = synth.make_workload(name)
    cfg = w.cfg
    B = cfg.num_seqs
    assert w.query.shape == (B, cfg.num_heads, cfg.head_dim)
    assert w.key_cache.shape == (w.num_blocks, 16, cfg.num_kv_heads, cfg.head_dim)
    lens = w.lens_np
    tables = w.tables_np
    assert tables.shape[1] * 16 >= lens.max()
    # logical blocks in use: distinct physical ids, except a beam group's shared prefix
    owners = {}
    for b in range(B):
        for j in range(blocks_for(int(lens[b]))):
            owners.setdefault(int(tables[b, j]), set()).add(b)
    if cfg.beams > 1:
        shared = [o for o in owners.values() if len(o) > 1]
        assert len(shared) == (B // cfg.beams) * cfg.prefix_len // 16
        assert all(len(o) == cfg.beams for o in shared)
    else:
        assert all(len(o) == 1 for o in owners.values())
    assert len(owners) == w.used_blocks
    # new-token slots are position L-1 of each sequence
    slots = w.slot_mapping.numpy()
    for b in range(B):
        assert slots[b] == slot_of(tables[b], int(lens[b]) - 1)
    # everything outside the cached tokens is NaN (16-bit caches) / 0x7F codes (FP8)
    if cfg.cache_dtype == "fp8_e4m3":
        assert np.all(bits_np(w.key_cache) == 0x7F)
        assert torch.isnan(w.k_scale).all()
        assert w.fill_slots.numel() == len(set(w.fill_slots.tolist()))
    else:
        kc = w.key_cache.float().numpy()
        cached = np.zeros((w.num_blocks, 16), dtype=bool)
        for b in range(B):
            for t in range(int(lens[b]) - 1):
                cached[tables[b, t // 16], t % 16] = True
        assert np.isnan(kc[~cached]).all()
        assert not np.isnan(kc[cached]).any()
        # table padding points only at never-written blocks
        for b in range(B):
            for j in range(blocks_for(int(lens[b])), tables.shape[1]):
                assert not cached[tables[b, j]].any()


def test_workloads_are_reproducible():
    a = synth.make_workload("tiny")
    b = synth.make_workload("tiny")
    for k, v in a.tensors().items():
        assert torch.equal(v.view(torch.uint8) if v.dtype != torch.uint8 else v,
                           b.tensors()[k].view(torch.uint8) if v.dtype != torch.uint8 else b.tensors()[k]), k


def test_lognormal_lengths_follow_the_recipe():
    cfg = synth.CONFIGS["gqa70b"]
    lens = synth.workloads.sample_lengths(cfg, np.random.default_rng(0))
    assert lens.min() >= 16 and lens.max() <= 4096 and lens.dtype == np.int32
