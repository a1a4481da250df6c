"""Pins of the oracle's codecs against torch's conversions, the OCP field table and closed forms."""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
ALL16 = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


def _same(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    both_nan = np.isnan(a) & np.isnan(b)
    eq = (a == b) & (np.signbit(a) == np.signbit(b))
    return bool(np.all(both_nan | eq))


def test_f16_decoder_matches_torch_and_numpy_on_all_patterns():
    ours = oracle.decode_f16(ALL16)
    t = torch.from_numpy(ALL16.view(np.int16)).view(torch.float16).to(torch.float64).numpy()
    n = ALL16.view(np.float16).astype(np.float64)
    assert _same(ours, t)
    assert _same(ours, n)


def test_bf16_decoder_matches_torch_on_all_patterns():
    ours = oracle.decode_bf16(ALL16)
    t = torch.from_numpy(ALL16.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert _same(ours, t)


def test_e4m3_table_matches_torch_on_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    t = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert _same(oracle.decode_e4m3(codes), t)
    tab = oracle.e4m3_table()
    assert np.isnan(tab).sum() == 2 and np.isnan(tab[0x7F]) and np.isnan(tab[0xFF])
    assert np.nanmax(tab) == 448.0 and np.nanmin(tab) == -448.0


def test_e4m3_golden_codes():
    with open(os.path.join(GOLDEN, "e4m3_ocp.json")) as f:
        fx = json.load(f)
    for code_s, val in ((c[0], c[1]) for c in fx["codes"]):
        code = int(code_s, 16)
        got = oracle.decode_e4m3(np.array([code], dtype=np.uint8))[0]
        if val == "nan":
            assert math.isnan(got), code_s
        else:
            assert got == val and math.copysign(1, got) == math.copysign(1, val), code_s


def test_e4m3_encode_roundtrips_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = oracle.decode_e4m3(codes).astype(np.float32)
    assert np.array_equal(oracle.encode_e4m3(vals), codes)


def test_e4m3_encode_ties_go_to_even_code():
    pos = oracle.e4m3_table()[:0x7F]
    mid = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)   # exact: 5 significant bits
    assert np.array_equal(mid.astype(np.float64), (pos[:-1] + pos[1:]) / 2)
    got = oracle.encode_e4m3(mid)
    lo = np.arange(0x7E)
    want = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(got, want.astype(np.uint8))
    # just off the midpoint, the nearer neighbour wins either way
    above = np.nextafter(mid, np.float32(np.inf))
    below = np.nextafter(mid, np.float32(-np.inf))
    assert np.array_equal(oracle.encode_e4m3(above), (lo + 1).astype(np.uint8))
    assert np.array_equal(oracle.encode_e4m3(below), lo.astype(np.uint8))


def test_e4m3_encode_saturates_and_keeps_sign():
    x = np.array([448.0, 449.0, 463.9, 464.0, 1e6, np.inf, -500.0, -np.inf, -0.0, 0.0, -1e-9, 1e-9],
                 dtype=np.float32)
    got = oracle.encode_e4m3(x)
    assert list(got) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x80, 0x00, 0x80, 0x00]


def test_e4m3_encode_matches_torch_on_every_bf16_pattern_in_range():
    x = torch.from_numpy(ALL16.view(np.int16)).view(torch.bfloat16).to(torch.float32)
    xf = x.numpy()
    keep = np.isfinite(xf) & (np.abs(xf) <= 448.0)
    ours = oracle.encode_e4m3(xf[keep])
    theirs = x[torch.from_numpy(keep)].to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, theirs)


def test_e4m3_encode_matches_torch_on_random_float32():
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.standard_normal(200_000).astype(np.float32) * np.float32(60.0),
        (rng.random(100_000) * 2 ** -5).astype(np.float32),     # subnormal range of E4M3
        rng.uniform(-448, 448, 100_000).astype(np.float32),
    ])
    x = np.clip(x, -448, 448).astype(np.float32)
    ours = oracle.encode_e4m3(x)
    theirs = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, theirs)


@pytest.mark.parametrize("dtype", ["f16", "bf16", "fp8_e4m3"])
def test_decode_bits_dispatch(dtype):
    bits = np.array([0, 1, 2], dtype=np.uint8 if dtype == "fp8_e4m3" else np.uint16)
    ref = {"f16": oracle.decode_f16, "bf16": oracle.decode_bf16, "fp8_e4m3": oracle.decode_e4m3}[dtype](bits)
    assert _same(oracle.decode_bits(bits, dtype), ref)
    with pytest.raises(ValueError):
        oracle.decode_bits(bits, "f32")
