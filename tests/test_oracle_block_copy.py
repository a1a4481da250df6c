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


def test_swap_matches_element_loop_across_pools():
    rng = np.random.default_rng(3)
    src = (_pool(rng, nb=9), _pool(rng, nb=9), None, None)
    dst = (_pool(rng, nb=5), _pool(rng, nb=5), None, None)
    pairs = np.array([[8, 0], [2, 4], [9, 1], [3, -1], [0, 5], [4, 3]], dtype=np.int64)
    k2, v2, _, _ = oracle.swap_blocks(src, dst, pairs)
    want_k, want_v = dst[0].copy(), dst[1].copy()
    for s_, d_ in pairs.tolist():
        if 0 <= s_ < 9 and 0 <= d_ < 5:
            for o in range(16):
                for h in range(src[0].shape[2]):
                    for e in range(src[0].shape[3]):
                        want_k[d_, o, h, e] = src[0][s_, o, h, e]
                        want_v[d_, o, h, e] = src[1][s_, o, h, e]
    assert np.array_equal(k2, want_k) and np.array_equal(v2, want_v)


def test_swap_out_then_in_restores_the_blocks_and_their_scales():
    rng = np.random.default_rng(4)
    gpu = (_pool(rng, nb=12, dtype=np.uint8), _pool(rng, nb=12, dtype=np.uint8),
           rng.random((12, 16)).astype(np.float32), rng.random((12, 16)).astype(np.float32))
    host = tuple(np.zeros((4,) + a.shape[1:], a.dtype) for a in gpu)
    out_pairs = np.array([[7, 0], [2, 1], [11, 2]])
    host2 = oracle.swap_blocks(gpu, host, out_pairs)
    back = oracle.swap_blocks(host2, gpu, np.array([[0, 3], [1, 4], [2, 5]]))
    for a, b in zip(gpu, back):
        for s_, d_ in [(7, 3), (2, 4), (11, 5)]:
            assert np.array_equal(b[d_], a[s_])
