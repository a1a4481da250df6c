"""Pins of the copy-on-write block copy oracle (CPU only).

The oracle is checked against an element-by-element Python loop over a tiny pool,
and against the invariants the definition fixes: destinations equal the sources'
prior contents, every other block and every source is unchanged, invalid pairs
and src == dst do nothing, and FP8 scales travel with their blocks.
"""

import numpy as np

import oracle


def _pool(rng, nb=7, hkv=2, d=4, dtype=np.uint16):
    hi = 256 if dtype == np.uint8 else 65536
    return rng.integers(0, hi, size=(nb, 16, hkv, d)).astype(dtype)


def test_copy_matches_element_loop():
    rng = np.random.default_rng(0)
    kc, vc = _pool(rng), _pool(rng)
    pairs = np.array([[1, 4], [2, 2], [0, 6], [-1, 3], [3, 7], [5, 0]], dtype=np.int64)
    k2, v2, _, _ = oracle.copy_blocks(kc, vc, pairs)
    want_k, want_v = kc.copy(), vc.copy()
    nb = kc.shape[0]
    for src, dst in pairs.tolist():
        if 0 <= src < nb and 0 <= dst < nb and src != dst:
            for o in range(16):
                for h in range(kc.shape[2]):
                    for e in range(kc.shape[3]):
                        want_k[dst, o, h, e] = kc[src, o, h, e]
                        want_v[dst, o, h, e] = vc[src, o, h, e]
    assert np.array_equal(k2, want_k) and np.array_equal(v2, want_v)


def test_copy_invariants_and_inputs_untouched():
    rng = np.random.default_rng(1)
    kc, vc = _pool(rng, nb=32), _pool(rng, nb=32)
    k0, v0 = kc.copy(), vc.copy()
    pairs = np.array([[3, 10], [4, 11], [5, 12], [40, 13], [6, -2], [7, 7]], dtype=np.int64)
    k2, v2, _, _ = oracle.copy_blocks(kc, vc, pairs)
    assert np.array_equal(kc, k0) and np.array_equal(vc, v0)          # arguments untouched
    for src, dst in [(3, 10), (4, 11), (5, 12)]:
        assert np.array_equal(k2[dst], k0[src]) and np.array_equal(v2[dst], v0[src])
    changed = {10, 11, 12}
    for b in range(32):
        if b not in changed:
            assert np.array_equal(k2[b], k0[b]) and np.array_equal(v2[b], v0[b])


def test_fp8_scales_travel_with_their_blocks():
    rng = np.random.default_rng(2)
    kc, vc = _pool(rng, dtype=np.uint8), _pool(rng, dtype=np.uint8)
    ks = rng.random((7, 16)).astype(np.float32)
    vs = rng.random((7, 16)).astype(np.float32)
    k2, v2, ks2, vs2 = oracle.copy_blocks(kc, vc, np.array([[0, 5]]), ks, vs)
    assert np.array_equal(ks2[5], ks[0]) and np.array_equal(vs2[5], vs[0])
    assert np.array_equal(np.delete(ks2, 5, 0), np.delete(ks, 5, 0))
    assert np.array_equal(k2[5], kc[0]) and np.array_equal(v2[5], vc[0])
