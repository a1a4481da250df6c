"""Host logic of the measurement: the bytes bench.py divides by the measured time.

The roofline numerator is the bytes the method must read per decode call: every cached
K and V row once (plus the FP8 per-token scales), the queries, the page-table entries of
the blocks in play and the lengths.  These tests recount them independently, from the
page tables themselves, on small and full-size synthetic workloads.
"""

import numpy as np
import pytest

import bench
import synth


def _recount(w, window=0, per_sequence=False):
    cfg = w.cfg
    eb = 1 if cfg.cache_dtype == "fp8_e4m3" else 2
    row = cfg.num_kv_heads * cfg.head_dim * eb            # one token's K (or V) over all KV heads
    slots, blocks = set(), 0
    for b, L in enumerate(w.lens_np):
        L = int(L)
        first = max(L - window, 0) if window else 0
        for t in range(first, L):
            phys = int(w.tables_np[b, t // 16])
            slots.add((b, phys, t % 16) if per_sequence else (phys, t % 16))
        blocks += (L + 15) // 16 - first // 16
    kv = len(slots) * (2 * row + (8 if eb == 1 else 0))
    q = cfg.num_seqs * cfg.num_heads * cfg.head_dim * 2
    return kv + q + blocks * 4 + cfg.num_seqs * 4


@pytest.mark.parametrize("name", ["tiny", "llama7b", "gqa70b"])
def test_algorithmic_bytes_count_every_cached_row_once(name):
    w = synth.make_workload(name)
    assert bench.algorithmic_bytes(w) == _recount(w)


def test_beams_unique_bytes_count_shared_prefix_blocks_once():
    w = synth.make_workload("fp8beams")
    cfg = w.cfg
    unique = bench.algorithmic_bytes(w)
    assert unique == _recount(w)                               # physical slots counted once
    assert bench.logical_bytes(w) == _recount(w, per_sequence=True)
    # 16 prompts x 1024 shared tokens + 64 beams x 256 private tokens, K and V of 8 x 128
    # one-byte codes plus two 4-byte scales per token, against 64 x 1280 tokens logically
    per_token = 8 * 128 * 2 + 8
    fixed = 64 * 32 * 128 * 2 + 64 * 80 * 4 + 64 * 4
    assert unique == (16 * 1024 + 64 * 256) * per_token + fixed
    assert bench.logical_bytes(w) == 64 * 1280 * per_token + fixed


@pytest.mark.parametrize("window", [1, 16, 17, 512])
def test_windowed_bytes_count_only_the_last_tokens_and_their_blocks(window):
    w = synth.make_workload("tiny")
    assert bench.algorithmic_bytes(w, window) == _recount(w, window=window)
    assert bench.algorithmic_bytes(w, window) <= bench.algorithmic_bytes(w)
    assert bench.algorithmic_bytes(w, 10 ** 6) == bench.algorithmic_bytes(w)
