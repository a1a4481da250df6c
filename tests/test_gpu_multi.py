"""GPU parity of multi-query paged attention (pa_decode_multi) against the float64 oracle.

The Q new tokens of a sequence are its last Q positions; the workload's own append
puts the last one in the cache, so the oracle and the GPU read the same caches.
"""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_187_amd as pa
import synth
from synth import bits_np

from gpu_cases import assert_close, gpu_append, oracle_caches, to_device

pytestmark = pytest.mark.gpu

LENS = (1, 2, 16, 17, 40, 100, 333, 1000)


def _case(q_len, hq, hkv, D=128, qd="bf16", cd="bf16", lens=LENS, seed=61):
    cfg = synth.DecodeConfig(name="multi", num_seqs=len(lens), num_heads=hq, num_kv_heads=hkv, head_dim=D,
                             q_dtype=qd, cache_dtype=cd, lengths="fixed", len_args=lens, seed=seed)
    wh = synth.make_workload(cfg)
    g = torch.Generator().manual_seed(seed + 7)
    tdt = torch.bfloat16 if qd == "bf16" else torch.float16
    q = torch.randn(len(lens), q_len, hq, D, generator=g).to(tdt)
    return cfg, wh, q


def _run(cfg, wh, q, part):
    kc, vc, ks, vs = oracle_caches(wh)
    ref = oracle.paged_decode_multi(bits_np(q), kc, vc, wh.tables_np, wh.lens_np, cfg.scale, cfg.q_dtype,
                                    cfg.cache_dtype, ks, vs)
    w = to_device(wh)
    gpu_append(w)
    qd = q.cuda()
    out = torch.empty_like(qd)
    pa.pa_decode_multi(out, qd, w.key_cache, w.value_cache, w.block_tables, w.context_lens, cfg.scale,
                       w.max_context_len, partition_size=part, k_scale=w.k_scale, v_scale=w.v_scale)
    torch.cuda.synchronize()
    return out, ref


@pytest.mark.parametrize("q_len", [1, 2, 3, 5, 16, 17, 40])
@pytest.mark.parametrize("hq,hkv,part", [(4, 4, 0), (8, 2, 32), (16, 2, 0), (12, 4, 0), (32, 1, 64)])
def test_multi_query_sweep(q_len, hq, hkv, part):
    print(f"[case] multi q_len={q_len} Hq={hq} Hkv={hkv} part={part}", flush=True)
    cfg, wh, q = _case(q_len, hq, hkv, seed=61 + q_len)
    out, ref = _run(cfg, wh, q, part)
    assert_close(out, ref, "bf16", f"multi Q={q_len} G={hq // hkv} part={part}")


@pytest.mark.parametrize("qd,cd,D,hq,hkv", [("f16", "f16", 64, 8, 8), ("bf16", "fp8_e4m3", 128, 8, 2),
                                          ("f16", "fp8_e4m3", 64, 4, 1)])
def test_multi_query_dtypes(qd, cd, D, hq, hkv):
    print(f"[case] multi dtypes q={qd} cache={cd} D={D} Hq={hq} Hkv={hkv}", flush=True)
    cfg, wh, q = _case(4, hq, hkv, D=D, qd=qd, cd=cd, seed=71)
    out, ref = _run(cfg, wh, q, 0)
    assert_close(out, ref, cd, f"multi dtypes {qd}/{cd} D={D}")


def test_multi_query_short_and_empty_sequences_give_zero_rows():
    print("[case] multi short/empty", flush=True)
    cfg, wh, q = _case(3, 8, 2, lens=(0, 1, 2, 3, 50), seed=81)
    out, ref = _run(cfg, wh, q, 0)
    assert_close(out, ref, "bf16", "multi short")
    assert torch.count_nonzero(out[0].float()) == 0 and torch.count_nonzero(out[1, :2].float()) == 0


def test_multi_query_of_one_token_matches_decode():
    print("[case] multi Q=1 vs pa_decode", flush=True)
    cfg, wh, q = _case(1, 8, 8, seed=91)
    w = to_device(wh)
    gpu_append(w)
    a = torch.empty_like(w.query)
    pa.pa_decode(a, q[:, 0].contiguous().cuda(), w.key_cache, w.value_cache, w.block_tables, w.context_lens,
                 cfg.scale, w.max_context_len)
    b = torch.empty(q.shape, dtype=q.dtype, device="cuda")
    pa.pa_decode_multi(b, q.cuda(), w.key_cache, w.value_cache, w.block_tables, w.context_lens, cfg.scale,
                       w.max_context_len)
    torch.cuda.synchronize()
    ref = oracle.paged_decode(bits_np(q[:, 0]), *oracle_caches(wh)[:2], wh.tables_np, wh.lens_np, cfg.scale,
                              cfg.q_dtype, cfg.cache_dtype)
    assert_close(a, ref, "bf16", "decode")
    assert_close(b[:, 0], ref, "bf16", "multi Q=1")
