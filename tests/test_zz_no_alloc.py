"""pa_decode_noalloc (partials in the library's fixed per-GPU scratch, nothing allocated) against
pa_decode with its own workspace, through the C ABI: bitwise equal outputs on two calls in a
row, the second with a smaller input, over both work splits and the VALU, matrix-core and FP8
paths; a call too large for the scratch is refused before anything is enqueued."""

import numpy as np
import pytest
import torch

import paged_kv_cache_187_amd as pa
import synth

from gpu_cases import assert_close, gpu_append, oracle_caches, oracle_decode, to_device

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[case] {msg}", flush=True)


def _cfg(**kw):
    base = dict(name="noalloc", num_seqs=6, num_heads=8, num_kv_heads=2, head_dim=128, q_dtype="bf16",
                cache_dtype="bf16", lengths="fixed", len_args=(700, 1, 0, 333, 2100, 17), seed=31)
    base.update(kw)
    return synth.DecodeConfig(**base)


def _both(w, part):
    """(pa_decode with a fresh workspace, pa_decode_noalloc) outputs of workload w (already appended)."""
    a = torch.empty_like(w.query)
    pa.pa_decode(a, w.query, w.key_cache, w.value_cache, w.block_tables, w.context_lens, w.cfg.scale,
                 w.max_context_len, partition_size=part, k_scale=w.k_scale, v_scale=w.v_scale)
    b = torch.full_like(w.query, float("nan"))
    pa.pa_decode_noalloc(b, w.query, w.key_cache, w.value_cache, w.block_tables, w.context_lens, w.cfg.scale,
                         w.max_context_len, partition_size=part, k_scale=w.k_scale, v_scale=w.v_scale)
    torch.cuda.synchronize()
    return a, b


CASES = [
    # (label, config overrides for the first call, config overrides for the second, smaller call, partition)
    ("gqa8 bf16 balanced", dict(), dict(num_seqs=3, len_args=(40, 5, 129), seed=32), 0),
    ("mha f16 fixed 64", dict(num_heads=4, num_kv_heads=4, q_dtype="f16", cache_dtype="f16"),
     dict(num_seqs=2, num_heads=4, num_kv_heads=4, q_dtype="f16", cache_dtype="f16", len_args=(200, 3), seed=33), 64),
    ("fp8 gqa4 balanced", dict(num_seqs=8, num_heads=8, num_kv_heads=2, cache_dtype="fp8_e4m3", lengths="beams",
                               len_args=(83,), beams=4, prefix_len=48),
     dict(num_seqs=4, num_heads=8, num_kv_heads=2, cache_dtype="fp8_e4m3", lengths="beams", len_args=(40,),
          beams=4, prefix_len=32, seed=34), 0),
]


@pytest.mark.parametrize("label,first,second,part", CASES, ids=[c[0] for c in CASES])
def test_noalloc_matches_pa_decode_on_two_calls(label, first, second, part):
    for k, over in enumerate((first, second)):
        cfg = _cfg(**over, partition_size=part)
        _say(f"noalloc {label} call {k + 1}: B={cfg.num_seqs} lens={cfg.len_args}")
        wh = synth.make_workload(cfg)
        w = to_device(wh)
        gpu_append(w)
        a, b = _both(w, part)
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"{label} call {k + 1}"
        assert_close(b, oracle_decode(wh, oracle_caches(wh)), cfg.cache_dtype, f"noalloc {label} call {k + 1}")


def test_noalloc_refuses_work_beyond_the_scratch():
    _say("noalloc refuses a workspace beyond the scratch")
    B, hq, hkv, d, L = 8, 64, 8, 128, 65536
    assert pa.decode_workspace_bytes(B, hq, hkv, d, L, 16) > (64 << 20)
    q = torch.zeros(B, hq, d, dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros(4, 16, hkv, d, dtype=torch.bfloat16, device="cuda")
    tables = torch.zeros(B, 1, dtype=torch.int32, device="cuda")
    lens = torch.zeros(B, dtype=torch.int32, device="cuda")
    out = torch.full_like(q, 7.0)
    with pytest.raises(pa.PagedAttnError) as e:
        pa.pa_decode_noalloc(out, q, kc, kc, tables, lens, 0.1, L, partition_size=16)
    assert e.value.status == 9
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())                       # nothing was enqueued
