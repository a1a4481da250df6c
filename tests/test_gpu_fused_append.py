"""pa_decode_append (the slot-mapped append fused into the decode) against pa_append_kv followed by
pa_decode: caches, FP8 scales and outputs bitwise equal, and the output within tolerance of the
oracle.  The synthetic workloads hold NaN in the new token's slot before the step, so an output
that read the slot instead of the new token's inputs would not be finite."""

import numpy as np
import pytest
import torch

import paged_kv_cache_187_amd as pa
import synth
from synth import bits_np

from gpu_cases import assert_close, oracle_caches, oracle_decode, to_device

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[case] {msg}", flush=True)


def _cfg(**kw):
    base = dict(name="fused", num_seqs=7, num_heads=4, num_kv_heads=4, head_dim=128, q_dtype="f16",
                cache_dtype="f16", lengths="fixed", len_args=(1, 16, 17, 0, 300, 33, 2050), seed=41)
    base.update(kw)
    return synth.DecodeConfig(**base)


def _fp8cfg(**kw):
    base = dict(name="fusedfp8", num_seqs=8, num_heads=8, num_kv_heads=2, head_dim=128, q_dtype="bf16",
                cache_dtype="fp8_e4m3", lengths="beams", len_args=(83,), seed=42, beams=4, prefix_len=48)
    base.update(kw)
    return synth.DecodeConfig(**base)


def _fill(w):
    """An FP8 workload's cached tokens, written by the quantising append (before the step)."""
    if w.fill_slots is not None and w.fill_slots.numel():
        pa.pa_append_kv(w.fill_key, w.fill_value, w.key_cache, w.value_cache, w.fill_slots, w.k_scale, w.v_scale)


def _state(w):
    return [bits_np(w.key_cache), bits_np(w.value_cache)] + \
        ([w.k_scale.cpu().numpy().view(np.uint32), w.v_scale.cpu().numpy().view(np.uint32)]
         if w.k_scale is not None else [])


def _compare(cfg, part=None, what=""):
    part = cfg.partition_size if part is None else part
    wh = synth.make_workload(cfg)
    a, b = to_device(wh), to_device(wh)
    for w in (a, b):
        _fill(w)
    out_a = torch.empty_like(a.query)
    pa.pa_append_kv(a.key_new, a.value_new, a.key_cache, a.value_cache, a.slot_mapping, a.k_scale, a.v_scale)
    pa.pa_decode(out_a, a.query, a.key_cache, a.value_cache, a.block_tables, a.context_lens, cfg.scale,
                 a.max_context_len, partition_size=part, k_scale=a.k_scale, v_scale=a.v_scale)
    out_b = torch.empty_like(b.query)
    pa.pa_decode_append(out_b, b.query, b.key_new, b.value_new, b.key_cache, b.value_cache, b.block_tables,
                        b.context_lens, cfg.scale, b.max_context_len, partition_size=part, k_scale=b.k_scale,
                        v_scale=b.v_scale)
    torch.cuda.synchronize()
    for x, y in zip(_state(a), _state(b)):
        assert np.array_equal(x, y), f"{what}: caches differ"
    assert torch.isfinite(out_b.float()).all(), f"{what}: the new token's slot leaked"
    assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16)), f"{what}: outputs differ"
    assert_close(out_b, oracle_decode(wh, oracle_caches(wh)), cfg.cache_dtype, f"fused {what}")
    return wh, out_b


SHAPES = [
    # (q dtype, cache dtype, Hq, Hkv, D, partition)
    ("f16", "f16", 4, 4, 128, 0),       # VALU, one head per wave
    ("bf16", "bf16", 8, 4, 64, 0),      # VALU, two heads per wave
    ("f16", "f16", 16, 2, 128, 0),      # matrix cores, groups of 8
    ("bf16", "bf16", 64, 2, 128, 0),    # groups of 32: two units of 16 heads share each KV head
    ("bf16", "bf16", 12, 4, 64, 48),    # groups of 3, fixed partitions
    ("f16", "f16", 2, 2, 64, 32),       # VALU, fixed partitions
]


@pytest.mark.parametrize("qd,cd,hq,hkv,D,part", SHAPES)
def test_fused_equals_append_then_decode(qd, cd, hq, hkv, D, part):
    _say(f"fused append {qd}/{cd} Hq={hq} Hkv={hkv} D={D} part={part}")
    cfg = _cfg(q_dtype=qd, cache_dtype=cd, num_heads=hq, num_kv_heads=hkv, head_dim=D, partition_size=part,
               seed=41 + hq + D)
    wh, out = _compare(cfg, what=f"{cd} G={hq // hkv} D={D} part={part}")
    # sequence 0 holds only the new token: its weight is exactly 1, so out = V bit for bit
    g = hq // hkv
    for h in range(hq):
        assert torch.equal(out[0, h].cpu().view(torch.int16), wh.value_new[0, h // g].view(torch.int16))


@pytest.mark.parametrize("qd,hq,hkv,D,part", [("bf16", 8, 2, 128, 0), ("f16", 4, 4, 64, 0), ("bf16", 8, 8, 128, 32),
                                              ("bf16", 16, 2, 128, 0)])
def test_fused_quantising_append(qd, hq, hkv, D, part):
    _say(f"fused FP8 append q={qd} Hq={hq} Hkv={hkv} D={D} part={part}")
    _compare(_fp8cfg(q_dtype=qd, num_heads=hq, num_kv_heads=hkv, head_dim=D, partition_size=part),
             what=f"fp8 G={hq // hkv} D={D} part={part}")


@pytest.mark.parametrize("name", ["llama7b", "gqa70b", "fp8beams"])
def test_fused_full_size(name):
    _say(f"fused append full-size {name}")
    _compare(synth.CONFIGS[name], what=f"{name} full")


def test_fused_skips_a_last_block_outside_the_pool():
    """A sequence whose last table entry is outside the pool: nothing is written and that block is
    not read, exactly as the separate append and decode do."""
    _say("fused append, last block outside the pool")
    cfg = _cfg(num_seqs=3, len_args=(40, 17, 5), seed=44)
    wh = synth.make_workload(cfg)
    wh.block_tables[1, 1] = wh.num_blocks + 5          # sequence 1's last block (tokens 16..16)
    wh.tables_np[1, 1] = wh.num_blocks + 5
    wh.slot_mapping[1] = -1                              # the separate append skips it too
    a, b = to_device(wh), to_device(wh)
    out_a, out_b = torch.empty_like(a.query), torch.empty_like(b.query)
    pa.pa_append_kv(a.key_new, a.value_new, a.key_cache, a.value_cache, a.slot_mapping)
    pa.pa_decode(out_a, a.query, a.key_cache, a.value_cache, a.block_tables, a.context_lens, cfg.scale,
                 a.max_context_len)
    pa.pa_decode_append(out_b, b.query, b.key_new, b.value_new, b.key_cache, b.value_cache, b.block_tables,
                        b.context_lens, cfg.scale, b.max_context_len)
    torch.cuda.synchronize()
    for x, y in zip(_state(a), _state(b)):
        assert np.array_equal(x, y)
    assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16))
