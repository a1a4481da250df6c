"""Pins of the paged decode oracle: brute force, library attention, invariants, closed forms."""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from synth import bits_np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
BS = 16


def _f16_bits(x):
    return torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.float16).view(torch.int16).numpy().view(np.uint16)


def _random_case(seed, B=3, Hq=4, Hkv=2, D=16, lens=(5, 16, 37), nb=12, dtype="f16"):
    rng = np.random.default_rng(seed)
    perm = rng.permutation(nb)
    tables = np.zeros((B, max(1, max(-(-n // BS) for n in lens))), dtype=np.int32)
    k = 0
    for b, n in enumerate(lens):
        for j in range(-(-n // BS)):
            tables[b, j] = perm[k]
            k += 1
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, Hq, D, generator=g).to(tdt).view(torch.int16).numpy().view(np.uint16)
    kc = torch.randn(nb, BS, Hkv, D, generator=g).to(tdt).view(torch.int16).numpy().view(np.uint16)
    vc = torch.randn(nb, BS, Hkv, D, generator=g).to(tdt).view(torch.int16).numpy().view(np.uint16)
    return q, kc, vc, tables, np.array(lens, dtype=np.int32)


def _dense_keys(kc, tables, b, L, dtype):
    dec = oracle.decode_bits(kc, dtype)
    return np.stack([dec[tables[b, t // BS], t % BS] for t in range(L)]) if L else np.zeros((0,) + dec.shape[2:])


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_matches_torch_sdpa_in_float64(dtype):
    q, kc, vc, tables, lens = _random_case(1, dtype=dtype)
    scale = 1 / math.sqrt(16)
    out = oracle.paged_decode(q, kc, vc, tables, lens, scale, dtype, dtype)
    qd = oracle.decode_bits(q, dtype)
    for b, L in enumerate(lens):
        K = torch.from_numpy(_dense_keys(kc, tables, b, L, dtype))        # [L, Hkv, D]
        V = torch.from_numpy(_dense_keys(vc, tables, b, L, dtype))
        Kh = K.permute(1, 0, 2).repeat_interleave(2, dim=0)[None]        # [1, Hq, L, D]
        Vh = V.permute(1, 0, 2).repeat_interleave(2, dim=0)[None]
        Q = torch.from_numpy(qd[b])[None, :, None, :]                     # [1, Hq, 1, D]
        ref = torch.nn.functional.scaled_dot_product_attention(Q, Kh, Vh, scale=scale)[0, :, 0].numpy()
        assert np.max(np.abs(out[b] - ref)) < 1e-12


def test_brute_force_python_loops_tiny():
    q, kc, vc, tables, lens = _random_case(2, B=2, Hq=2, Hkv=1, D=4, lens=(3, 18), nb=5)
    scale = 0.7
    out = oracle.paged_decode(q, kc, vc, tables, lens, scale, "f16", "f16")
    qd, kd, vd = (oracle.decode_f16(a) for a in (q, kc, vc))
    for b in range(2):
        for h in range(2):
            L = int(lens[b])
            s = []
            for t in range(L):
                p = tables[b, t // BS]
                s.append(scale * sum(qd[b, h, e] * kd[p, t % BS, 0, e] for e in range(4)))
            m = max(s)
            w = [math.exp(x - m) for x in s]
            tot = sum(w)
            for e in range(4):
                ref = sum(w[t] * vd[tables[b, t // BS], t % BS, 0, e] for t in range(L)) / tot
                assert abs(out[b, h, e] - ref) < 1e-12


def test_permuting_physical_blocks_leaves_output_bitwise_identical():
    q, kc, vc, tables, lens = _random_case(3, lens=(40, 1, 33), nb=20)
    out = oracle.paged_decode(q, kc, vc, tables, lens, 0.25, "f16", "f16")
    rng = np.random.default_rng(9)
    perm = rng.permutation(kc.shape[0])          # new physical id of old block i is perm[i]
    kc2 = np.empty_like(kc)
    vc2 = np.empty_like(vc)
    kc2[perm] = kc
    vc2[perm] = vc
    tables2 = perm[tables].astype(np.int32)
    out2 = oracle.paged_decode(q, kc2, vc2, tables2, lens, 0.25, "f16", "f16")
    assert np.array_equal(out, out2)


def test_softmax_weights_sum_to_one_and_single_token_returns_v():
    rng = np.random.default_rng(4)
    q = rng.standard_normal(32)
    K = rng.standard_normal((300, 32)) * 3
    w = oracle.attention_weights(q, K, 0.2)
    assert abs(w.sum() - 1.0) < 1e-12 and np.all(w >= 0)
    # one cached token: its weight is exactly 1, so the output is its V row exactly
    q, kc, vc, tables, lens = _random_case(5, lens=(1, 1, 1))
    out = oracle.paged_decode(q, kc, vc, tables, lens, 0.3, "f16", "f16")
    vd = oracle.decode_f16(vc)
    for b in range(3):
        for h in range(4):
            assert np.array_equal(out[b, h], vd[tables[b, 0], 0, h // 2])


def test_constant_v_and_equal_keys():
    q, kc, vc, tables, lens = _random_case(6, lens=(20, 7, 33))
    vc_const = np.broadcast_to(_f16_bits(np.linspace(-2, 2, 16)), vc.shape).copy()
    out = oracle.paged_decode(q, kc, vc_const, tables, lens, 0.5, "f16", "f16")
    assert np.max(np.abs(out - oracle.decode_f16(vc_const[0, 0, 0]))) < 1e-14
    kc_eq = np.broadcast_to(_f16_bits(np.full(16, 0.3)), kc.shape).copy()
    out = oracle.paged_decode(q, kc_eq, vc, tables, lens, 0.5, "f16", "f16")
    vd = oracle.decode_f16(vc)
    for b, L in enumerate(lens):
        V = np.stack([vd[tables[b, t // BS], t % BS] for t in range(L)])
        for h in range(4):
            assert np.max(np.abs(out[b, h] - V[:, h // 2].mean(0))) < 1e-13


def test_gqa_equals_mha_with_repeated_kv_heads():
    q, kc, vc, tables, lens = _random_case(7, Hq=8, Hkv=2, lens=(17, 50, 3), nb=16)
    out = oracle.paged_decode(q, kc, vc, tables, lens, 0.25, "f16", "f16")
    kc_rep = np.repeat(kc, 4, axis=2)
    vc_rep = np.repeat(vc, 4, axis=2)
    out_mha = oracle.paged_decode(q, kc_rep, vc_rep, tables, lens, 0.25, "f16", "f16")
    assert np.array_equal(out, out_mha)


@pytest.mark.parametrize("part", [1, 5, 16, 32, 64])
def test_partition_merge_equals_unsplit(part):
    rng = np.random.default_rng(8)
    q = rng.standard_normal(64)
    K = rng.standard_normal((203, 64))
    V = rng.standard_normal((203, 64))
    full = oracle.attend(q, K, V, 0.125)
    parts = [oracle.partial_attend(q, K[i:i + part], V[i:i + part], 0.125) for i in range(0, 203, part)]
    parts.append(oracle.partial_attend(q, K[:0], V[:0], 0.125))   # an empty partition changes nothing
    assert np.max(np.abs(oracle.merge_partials(parts) - full)) < 1e-12


def test_nan_outside_the_context_never_reaches_the_output():
    q, kc, vc, tables, lens = _random_case(10, lens=(5, 16, 37), nb=12)
    used = {(int(tables[b, t // BS]), t % BS) for b, L in enumerate(lens) for t in range(L)}
    kc2, vc2 = kc.copy(), vc.copy()
    for blk in range(kc.shape[0]):
        for off in range(BS):
            if (blk, off) not in used:
                kc2[blk, off] = 0x7E00
                vc2[blk, off] = 0x7E00
    a = oracle.paged_decode(q, kc, vc, tables, lens, 0.25, "f16", "f16")
    b = oracle.paged_decode(q, kc2, vc2, tables, lens, 0.25, "f16", "f16")
    assert np.array_equal(a, b)


def test_fp8_cache_applies_per_token_scales():
    rng = np.random.default_rng(12)
    nb, Hkv, D = 4, 2, 8
    kc = rng.integers(0, 0x7E, size=(nb, BS, Hkv, D)).astype(np.uint8)
    vc = rng.integers(0x80, 0xFE, size=(nb, BS, Hkv, D)).astype(np.uint8)
    ks = rng.uniform(0.01, 0.1, size=(nb, BS)).astype(np.float32)
    vs = rng.uniform(0.01, 0.1, size=(nb, BS)).astype(np.float32)
    q = torch.randn(1, 4, D, generator=torch.Generator().manual_seed(1)).to(torch.bfloat16)
    qb = q.view(torch.int16).numpy().view(np.uint16)
    tables = np.array([[2, 0]], dtype=np.int32)
    lens = np.array([20], dtype=np.int32)
    out = oracle.paged_decode(qb, kc, vc, tables, lens, 0.3, "bf16", "fp8_e4m3", ks, vs)
    tab = oracle.e4m3_table()
    qd = q.to(torch.float64).numpy()[0]
    for h in range(4):
        K = np.stack([tab[kc[tables[0, t // BS], t % BS, h // 2]] * np.float64(ks[tables[0, t // BS], t % BS])
                      for t in range(20)])
        V = np.stack([tab[vc[tables[0, t // BS], t % BS, h // 2]] * np.float64(vs[tables[0, t // BS], t % BS])
                      for t in range(20)])
        s = 0.3 * K @ qd[h]
        w = np.exp(s - s.max())
        ref = (w / w.sum()) @ V
        assert np.max(np.abs(out[0, h] - ref)) < 1e-13


def test_paged_decode_one_matches_batch():
    q, kc, vc, tables, lens = _random_case(13, lens=(30, 9, 1), nb=8)
    out = oracle.paged_decode(q, kc, vc, tables, lens, 0.25, "f16", "f16")
    qd = oracle.decode_f16(q)
    for b in range(3):
        for h in range(4):
            one = oracle.paged_decode_one(qd[b, h], kc, vc, tables[b], int(lens[b]), h // 2, 0.25, "f16")
            assert np.array_equal(one, out[b, h])


def _golden_inputs(case):
    D, Hq, Hkv, nb = case["head_dim"], case["num_heads"], case["num_kv_heads"], case["num_blocks"]
    L = case["context_len"]
    if isinstance(case["tokens_k"], str):
        ks = [[[1.0, 1.0]] for _ in range(L)]
        vs = [[[float(t), float(2 * t)]] for t in range(L)]
    else:
        ks, vs = case["tokens_k"], case["tokens_v"]
    kc = np.full((nb, BS, Hkv, D), 0x7E00, dtype=np.uint16)    # NaN everywhere else
    vc = kc.copy()
    table = case["block_table"]
    for t in range(L):
        kc[table[t // BS], t % BS] = _f16_bits(ks[t])
        vc[table[t // BS], t % BS] = _f16_bits(vs[t])
    q = _f16_bits(case["q"]).reshape(1, Hq, D)
    scale = math.log(3.0) if case["scale"] == "ln3" else float(case["scale"])
    return q, kc, vc, np.array([table], dtype=np.int32), np.array([L], dtype=np.int32), scale


def test_golden_worked_examples():
    with open(os.path.join(GOLDEN, "paged_attention_worked.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        q, kc, vc, tables, lens, scale = _golden_inputs(case)
        out = oracle.paged_decode(q, kc, vc, tables, lens, scale, "f16", "f16")
        assert np.max(np.abs(out[0] - np.array(case["expected"]))) < 1e-12, case["name"]


def test_synth_tiny_workload_through_oracle_is_finite():
    w = synth.make_workload("tiny")
    kc, vc = oracle.append_kv(bits_np(w.key_cache), bits_np(w.value_cache), bits_np(w.key_new),
                              bits_np(w.value_new), w.slot_mapping.numpy())
    out = oracle.paged_decode(bits_np(w.query), kc, vc, w.tables_np, w.lens_np, w.cfg.scale, "f16", "f16")
    assert np.all(np.isfinite(out))
    # sequence 0 has one token, the one appended this step: its output is that token's V row
    vd = oracle.decode_f16(bits_np(w.value_new))
    assert np.array_equal(out[0], vd[0])


@pytest.mark.parametrize("window", [0, 37, 38, 1000])
def test_window_covering_the_context_changes_nothing(window):
    q, kc, vc, tables, lens = _random_case(31)
    full = oracle.paged_decode(q, kc, vc, tables, lens, 0.25, "f16", "f16")
    win = oracle.paged_decode(q, kc, vc, tables, lens, 0.25, "f16", "f16", window=window)
    assert np.array_equal(full, win)


def test_window_of_one_returns_the_last_v_row():
    q, kc, vc, tables, lens = _random_case(32)
    out = oracle.paged_decode(q, kc, vc, tables, lens, 0.25, "f16", "f16", window=1)
    for b, L in enumerate(lens):
        last = oracle.decode_bits(vc, "f16")[tables[b, (L - 1) // BS], (L - 1) % BS]
        for h in range(q.shape[1]):
            assert np.array_equal(out[b, h], last[h // 2])


@pytest.mark.parametrize("window", [2, 5, 16, 17, 20])
def test_window_equals_dense_attention_over_the_last_tokens(window):
    """Python loops over the last W tokens of each sequence, written out directly."""
    q, kc, vc, tables, lens = _random_case(33, lens=(5, 16, 37))
    out = oracle.paged_decode(q, kc, vc, tables, lens, 0.3, "f16", "f16", window=window)
    qd = oracle.decode_bits(q, "f16")
    kd, vd = oracle.decode_bits(kc, "f16"), oracle.decode_bits(vc, "f16")
    for b, L in enumerate(lens):
        toks = list(range(max(0, L - window), L))
        for h in range(qd.shape[1]):
            hk = h // 2
            s = [0.3 * sum(qd[b, h, d] * kd[tables[b, t // BS], t % BS, hk, d] for d in range(qd.shape[2]))
                 for t in toks]
            mx = max(s)
            e = [math.exp(x - mx) for x in s]
            want = [sum(e[i] * vd[tables[b, t // BS], t % BS, hk, d] for i, t in enumerate(toks)) / sum(e)
                    for d in range(qd.shape[2])]
            assert np.allclose(out[b, h], want, rtol=1e-12, atol=1e-12)


def test_tokens_before_the_window_never_reach_the_output():
    q, kc, vc, tables, lens = _random_case(34, lens=(40, 33, 50))
    window = 9
    clean = oracle.paged_decode(q, kc, vc, tables, lens, 0.25, "f16", "f16", window=window)
    kp, vp = kc.copy(), vc.copy()
    for b, L in enumerate(lens):
        for t in range(0, L - window):
            kp[tables[b, t // BS], t % BS] = 0x7E00
            vp[tables[b, t // BS], t % BS] = 0x7E00
    poisoned = oracle.paged_decode(q, kp, vp, tables, lens, 0.25, "f16", "f16", window=window)
    assert np.array_equal(clean, poisoned) and np.isfinite(poisoned).all()


def _multi_case(seed, B=3, Q=4, Hq=4, Hkv=2, D=16, lens=(5, 16, 37), nb=12):
    q1, kc, vc, tables, lens_np = _random_case(seed, B=B, Hq=Hq, Hkv=Hkv, D=D, lens=lens, nb=nb)
    g = torch.Generator().manual_seed(seed + 100)
    q = torch.randn(B, Q, Hq, D, generator=g).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    return q, kc, vc, tables, lens_np


def test_multi_query_of_one_token_is_plain_decode():
    q, kc, vc, tables, lens = _multi_case(51, Q=1)
    multi = oracle.paged_decode_multi(q, kc, vc, tables, lens, 0.25, "f16", "f16")
    single = oracle.paged_decode(q[:, 0], kc, vc, tables, lens, 0.25, "f16", "f16")
    assert np.array_equal(multi[:, 0], single)


def test_multi_query_causal_python_loops():
    """Token i of the new chunk attends to positions 0 .. L - Q + i, written out directly."""
    Q = 5
    q, kc, vc, tables, lens = _multi_case(52, Q=Q, lens=(5, 16, 37))
    out = oracle.paged_decode_multi(q, kc, vc, tables, lens, 0.3, "f16", "f16")
    qd = oracle.decode_bits(q, "f16")
    kd, vd = oracle.decode_bits(kc, "f16"), oracle.decode_bits(vc, "f16")
    for b, L in enumerate(lens):
        for i in range(Q):
            toks = list(range(0, L - Q + i + 1))
            for h in range(qd.shape[2]):
                hk = h // 2
                if not toks:
                    assert np.array_equal(out[b, i, h], np.zeros(qd.shape[3]))
                    continue
                s = [0.3 * sum(qd[b, i, h, d] * kd[tables[b, t // BS], t % BS, hk, d] for d in range(qd.shape[3]))
                     for t in toks]
                mx = max(s)
                e = [math.exp(x - mx) for x in s]
                want = [sum(e[k] * vd[tables[b, t // BS], t % BS, hk, d] for k, t in enumerate(toks)) / sum(e)
                        for d in range(qd.shape[3])]
                assert np.allclose(out[b, i, h], want, rtol=1e-12, atol=1e-12)


def test_multi_query_matches_torch_sdpa_with_offset_causal_mask():
    """torch's scaled_dot_product_attention in float64 with the mask t <= L - Q + i."""
    Q = 6
    q, kc, vc, tables, lens = _multi_case(53, Q=Q, lens=(9, 16, 40), Hq=6, Hkv=3)
    out = oracle.paged_decode_multi(q, kc, vc, tables, lens, 0.2, "f16", "f16")
    qd = torch.from_numpy(oracle.decode_bits(q, "f16"))
    for b, L in enumerate(lens):
        K = torch.from_numpy(_dense_keys(kc, tables, b, L, "f16"))          # [L, Hkv, D]
        V = torch.from_numpy(_dense_keys(vc, tables, b, L, "f16"))
        mask = torch.tensor([[t <= L - Q + i for t in range(L)] for i in range(Q)])
        for h in range(6):
            ref = torch.nn.functional.scaled_dot_product_attention(
                qd[b, :, h][None], K[:, h // 2][None], V[:, h // 2][None], attn_mask=mask[None], scale=0.2)[0]
            assert np.allclose(out[b, :, h], ref.numpy(), rtol=1e-12, atol=1e-12)
