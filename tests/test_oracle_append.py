"""Pins of the oracle's slot-mapped append and its per-token FP8 quantiser."""

import numpy as np
import pytest
import torch

import oracle
from oracle.codecs import e4m3_table

BS = 16


def _pools(rng, nb, hkv, d, dtype=np.uint16):
    k = rng.integers(0, 1 << 16, size=(nb, BS, hkv, d)).astype(dtype)
    v = rng.integers(0, 1 << 16, size=(nb, BS, hkv, d)).astype(dtype)
    return k, v


def test_append_matches_elementwise_loop_and_leaves_other_slots():
    rng = np.random.default_rng(0)
    nb, hkv, d, T = 6, 2, 8, 7
    kc, vc = _pools(rng, nb, hkv, d)
    k = rng.integers(0, 1 << 16, size=(T, hkv, d)).astype(np.uint16)
    v = rng.integers(0, 1 << 16, size=(T, hkv, d)).astype(np.uint16)
    slots = np.array([0, 15, 16, -1, 95, 96, -7], dtype=np.int64)   # 96 = 6 * 16: past the pool
    nk, nv = oracle.append_kv(kc, vc, k, v, slots)
    ek, ev = kc.copy(), vc.copy()
    for t in range(T):
        s = int(slots[t])
        if s < 0 or s >= nb * BS:
            continue
        for h in range(hkv):
            for e in range(d):
                ek[s // BS, s % BS, h, e] = k[t, h, e]
                ev[s // BS, s % BS, h, e] = v[t, h, e]
    assert np.array_equal(nk, ek) and np.array_equal(nv, ev)
    # arguments untouched, untouched slots identical
    written = {int(s) for s in slots if 0 <= s < nb * BS}
    for blk in range(nb):
        for off in range(BS):
            if blk * BS + off not in written:
                assert np.array_equal(nk[blk, off], kc[blk, off])


def test_quantiser_amax_maps_to_448_and_error_within_half_ulp():
    x_bf16 = torch.randn(64, 1024, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    x = x_bf16.to(torch.float32).numpy()
    codes, scales = oracle.quantize_tokens_e4m3(x)
    tab = e4m3_table()
    deq = tab[codes] * scales[:, None].astype(np.float64)
    amax_idx = np.argmax(np.abs(x), axis=1)
    for t in range(x.shape[0]):
        c = codes[t, amax_idx[t]]
        assert c in (0x7E, 0xFE)
        assert scales[t] == np.float32(np.max(np.abs(x[t]))) / np.float32(448.0)
    # |deq - x| <= half the E4M3 spacing at |x/scale|, times scale (+ the float32 division's rounding)
    y = np.abs(x / scales[:, None].astype(np.float64))
    e = np.floor(np.log2(np.maximum(y, 2.0 ** -6)))
    half_ulp = 0.5 * 2.0 ** (e - 3)
    bound = (half_ulp + y * 2.0 ** -24) * scales[:, None]
    assert np.all(np.abs(deq - x) <= bound + 1e-30)


def test_quantiser_zero_row_and_signs():
    x = np.zeros((2, 8), dtype=np.float32)
    x[1] = -0.0
    codes, scales = oracle.quantize_tokens_e4m3(x)
    assert list(scales) == [1.0, 1.0]
    assert np.all(codes[0] == 0x00) and np.all(codes[1] == 0x80)
    x = np.array([[1.0, -2.0, 0.5, -0.25]], dtype=np.float32)
    codes, scales = oracle.quantize_tokens_e4m3(x)
    assert scales[0] == np.float32(2.0) / np.float32(448.0)
    # x/scale ~ [224, -448, 112, -56] = 1.75 * 2^[7, 8, 6, 5]: fraction 6, exponent fields 14, 15, 13, 12
    assert list(codes[0]) == [0x76, 0xFE, 0x6E, 0xE6]


def test_quantiser_agrees_with_torch_conversion_of_the_scaled_values():
    g = torch.Generator().manual_seed(11)
    x = (torch.randn(128, 512, generator=g) * 3).to(torch.bfloat16).to(torch.float32)
    codes, scales = oracle.quantize_tokens_e4m3(x.numpy())
    y = x / torch.from_numpy(scales)[:, None]          # float32 division, as specified
    ref = y.clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref)


def _torch_quantise(x):
    """Per-token E4M3 codes and scales computed with torch alone (not the oracle's encoder):
    amax and the float32 division by 448 in torch, then torch's own E4M3 conversion of the
    float32 quotients, clamped to +-448 first (torch's conversion gives NaN past 464)."""
    x = x.to(torch.float32)
    amax = x.abs().amax(dim=1)
    sc = torch.where(amax == 0, torch.ones_like(amax), amax / torch.tensor(448.0))
    y = (x / sc[:, None]).clamp(-448, 448)
    return y.to(torch.float8_e4m3fn).view(torch.uint8).numpy(), sc.numpy()


@pytest.mark.parametrize("src", ["bf16", "f16"])
def test_fp8_append_scatter_writes_codes_and_scales(src):
    """Both halves of the quantising append: K codes and scales from K, V codes and scales from
    V (drawn apart so that a swapped operand fails), every other slot and scale unchanged,
    slots past the pool (16 * num_blocks and above) and negative slots skipped."""
    nb, hkv, d, T = 4, 2, 16, 7
    tdt = torch.bfloat16 if src == "bf16" else torch.float16
    kc = np.full((nb, BS, hkv, d), 0x7F, dtype=np.uint8)
    vc = np.full((nb, BS, hkv, d), 0x7F, dtype=np.uint8)
    ks = np.full((nb, BS), np.nan, dtype=np.float32)
    vs = np.full((nb, BS), np.nan, dtype=np.float32)
    k = torch.randn(T, hkv, d, generator=torch.Generator().manual_seed(1)).to(tdt)
    v = (torch.randn(T, hkv, d, generator=torch.Generator().manual_seed(2)) * 5).to(tdt)
    v[2] = 0                                          # an all-zero V row: scale 1, codes 0
    kb = k.view(torch.int16).numpy().view(np.uint16)
    vb = v.view(torch.int16).numpy().view(np.uint16)
    slots = np.array([3, -1, 17, 63, 32, nb * BS, nb * BS + 5], dtype=np.int64)
    nk, nv, nks, nvs = oracle.append_kv_e4m3(kc, vc, ks, vs, kb, vb, src, slots)
    qk, sk = _torch_quantise(k.reshape(T, -1))
    qv, sv = _torch_quantise(v.reshape(T, -1))
    assert not np.array_equal(qk, qv) and not np.array_equal(sk, sv)
    assert sv[2] == 1.0 and np.all(qv[2] == 0)
    written = np.zeros((nb, BS), dtype=bool)
    for t, s in enumerate(slots):
        if s < 0 or s >= nb * BS:
            continue
        blk, off = divmod(int(s), BS)
        written[blk, off] = True
        assert np.array_equal(nk[blk, off].reshape(-1), qk[t]), f"K codes of token {t}"
        assert np.array_equal(nv[blk, off].reshape(-1), qv[t]), f"V codes of token {t}"
        assert nks[blk, off].view(np.uint32) == sk[t].view(np.uint32), f"K scale of token {t}"
        assert nvs[blk, off].view(np.uint32) == sv[t].view(np.uint32), f"V scale of token {t}"
    assert written.sum() == 4
    for pool in (nk, nv):
        assert np.all(pool[~written] == 0x7F)
    for sc in (nks, nvs):
        assert np.all(np.isnan(sc[~written]))
    # the arguments are left as they were
    assert np.all(kc == 0x7F) and np.all(vc == 0x7F) and np.isnan(ks).all() and np.isnan(vs).all()
