"""GPU parity of paged decode attention against the float64 oracle."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_187_amd as pa
import synth

from gpu_cases import (assert_close, gpu_append, gpu_decode, gpu_step, oracle_caches, oracle_decode,
                       sequence_reference, to_device)

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[case] {msg}", flush=True)


def _cfg(**kw):
    base = dict(name="sweep", num_seqs=5, num_heads=4, num_kv_heads=4, head_dim=128, q_dtype="f16",
                cache_dtype="f16", lengths="fixed", len_args=(1, 15, 16, 17, 100), seed=5)
    base.update(kw)
    return synth.DecodeConfig(**base)


def _run_and_check(cfg, partition_size=None, what=""):
    wh = synth.make_workload(cfg)
    w = to_device(wh)
    out = gpu_step(w, partition_size)
    ref = oracle_decode(wh, oracle_caches(wh))
    assert_close(out, ref, cfg.cache_dtype, what or cfg.name)
    return w, wh, out, ref


def test_tiny_config():
    _say("tiny config")
    w, wh, out, ref = _run_and_check(synth.CONFIGS["tiny"])
    # sequence 0 holds only this step's token: its weight is exactly 1, so out = V bit for bit
    assert torch.equal(out[0].cpu().view(torch.int16), wh.value_new[0].view(torch.int16))


SWEEP = [
    # (D, q dtype, cache dtype, Hq, Hkv, lengths, partition)
    (128, "f16", "f16", 4, 4, (1, 15, 16, 17, 100), 0),
    (64, "f16", "f16", 4, 4, (1, 15, 16, 17, 100), 0),
    (128, "bf16", "bf16", 8, 1, (33, 2, 64, 65, 300), 0),
    (64, "bf16", "bf16", 16, 2, (31, 32, 47, 48, 49), 16),
    (128, "f16", "f16", 8, 2, (1, 15, 16, 17, 100), 32),
    (128, "bf16", "bf16", 12, 4, (200, 15, 513, 17, 1), 64),
    (64, "f16", "f16", 6, 2, (5, 0, 1024, 1023, 1025), 512),
    (128, "f16", "f16", 2, 1, (0, 0, 3, 0, 0), 0),
    (128, "bf16", "bf16", 64, 8, (1500, 16, 4096, 700, 33), 512),
    (128, "f16", "f16", 32, 32, (2048, 1, 999, 16, 17), 256),
    (64, "f16", "f16", 5, 5, (40, 41, 42, 43, 44), 48),
]


@pytest.mark.parametrize("D,qd,cd,hq,hkv,lens,part", SWEEP)
def test_shape_sweep(D, qd, cd, hq, hkv, lens, part):
    _say(f"sweep D={D} {qd}/{cd} Hq={hq} Hkv={hkv} lens={lens} part={part}")
    cfg = _cfg(head_dim=D, q_dtype=qd, cache_dtype=cd, num_heads=hq, num_kv_heads=hkv, len_args=lens,
               partition_size=part, seed=D + hq + hkv + part)
    _run_and_check(cfg, what=f"D={D} {cd} G={hq // hkv} part={part}")


def _fp8cfg(**kw):
    base = dict(name="fp8sweep", num_seqs=8, num_heads=8, num_kv_heads=2, head_dim=128, q_dtype="bf16",
                cache_dtype="fp8_e4m3", lengths="beams", len_args=(83,), seed=77, beams=4, prefix_len=48)
    base.update(kw)
    return synth.DecodeConfig(**base)


@pytest.mark.parametrize("qd,D,hq,hkv,part", [("bf16", 128, 8, 2, 0), ("f16", 64, 4, 4, 32),
                                              ("bf16", 128, 16, 2, 16), ("bf16", 64, 8, 8, 0)])
def test_fp8_cache_sweep(qd, D, hq, hkv, part):
    _say(f"fp8 D={D} q={qd} Hq={hq} Hkv={hkv} part={part}")
    cfg = _fp8cfg(q_dtype=qd, head_dim=D, num_heads=hq, num_kv_heads=hkv, partition_size=part)
    _run_and_check(cfg, what=f"fp8 D={D} G={hq // hkv} part={part}")


@pytest.mark.parametrize("hq,hkv", [(8, 2), (4, 4)])
def test_fp8_scales_need_only_4_byte_alignment(hq, hkv):
    """FP8 per-token scales at a 4-byte (not 16-byte) offset, on both decode paths (matrix cores
    for G = 4, VALU for G = 1): the decode reads each scale with its own 4-byte load."""
    _say(f"fp8 scales at a 4-byte offset Hq={hq} Hkv={hkv}")
    cfg = _fp8cfg(num_heads=hq, num_kv_heads=hkv)
    wh = synth.make_workload(cfg)
    w = to_device(wh)
    gpu_append(w)
    shifted = []
    for sc in (w.k_scale, w.v_scale):
        buf = torch.empty(sc.numel() + 4, dtype=torch.float32, device=sc.device)
        view = buf[1:1 + sc.numel()].view_as(sc)
        view.copy_(sc)
        assert view.data_ptr() % 16 == 4
        shifted.append(view)
    out = torch.empty_like(w.query)
    pa.pa_decode(out, w.query, w.key_cache, w.value_cache, w.block_tables, w.context_lens, cfg.scale,
                 w.max_context_len, partition_size=cfg.partition_size, k_scale=shifted[0], v_scale=shifted[1])
    torch.cuda.synchronize()
    assert_close(out, oracle_decode(wh, oracle_caches(wh)), cfg.cache_dtype, f"fp8 scales +4 bytes G={hq // hkv}")


@pytest.mark.parametrize("qd,D,hq", [("bf16", 128, 1), ("bf16", 128, 4), ("f16", 128, 4), ("bf16", 64, 4),
                                     ("f16", 64, 8)])
def test_fp8_every_code_through_single_token_contexts(qd, D, hq):
    """L = 1: the weight is exactly 1, so out = decode(V code) * v_scale, exact in the query type.

    hq query heads share the one KV head: hq = 1 takes the VALU path, 4 and 8 the matrix-core path.
    """
    _say(f"fp8 every code, single-token contexts, q={qd} D={D} heads={hq}")
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    hkv = 1
    B = -(-codes.size // D)
    vc = np.zeros((B, 16, hkv, D), dtype=np.uint8)
    flat = np.zeros(B * D, dtype=np.uint8)
    flat[:codes.size] = codes
    vc[:, 0, 0, :] = flat.reshape(B, D)
    kc = np.full_like(vc, 0x38)          # 1.0
    vc[:, 1:] = 0x7F                     # NaN past the context
    ks = np.ones((B, 16), np.float32)
    vs = np.ones((B, 16), np.float32)
    vs[:, 1:] = np.nan
    tdt = torch.bfloat16 if qd == "bf16" else torch.float16
    q = torch.randn(B, hq, D, generator=torch.Generator().manual_seed(0)).to(tdt).cuda()
    out = torch.empty_like(q)
    tables = torch.arange(B, dtype=torch.int32).view(B, 1).cuda()
    lens = torch.ones(B, dtype=torch.int32).cuda()
    pa.pa_decode(out, q, torch.from_numpy(kc).cuda(), torch.from_numpy(vc).cuda(), tables, lens, 0.1, 1,
                 k_scale=torch.from_numpy(ks).cuda(), v_scale=torch.from_numpy(vs).cuda())
    torch.cuda.synchronize()
    want = oracle.decode_e4m3(codes)
    for h in range(hq):
        got = out[:, h].cpu().to(torch.float64).numpy().reshape(-1)[:codes.size]
        assert np.array_equal(got, want), f"head {h}"


def test_poison_never_reaches_the_output_and_runs_are_deterministic():
    _say("poison + determinism")
    cfg = _cfg(num_heads=8, num_kv_heads=2, len_args=(3, 16, 250, 17, 64), partition_size=32)
    wh = synth.make_workload(cfg)
    w = to_device(wh)
    a = gpu_step(w)
    b = gpu_decode(w)
    torch.cuda.synchronize()
    assert torch.isfinite(a.float()).all()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_permuting_physical_blocks_is_bitwise_invisible():
    _say("permutation invariance")
    cfg = _cfg(num_heads=8, num_kv_heads=2, len_args=(40, 1, 33, 200, 16), partition_size=64, seed=9)
    wh = synth.make_workload(cfg)
    w = to_device(wh)
    a = gpu_step(w)
    perm = torch.from_numpy(np.random.default_rng(3).permutation(wh.num_blocks)).cuda()
    kc2 = torch.empty_like(w.key_cache)
    vc2 = torch.empty_like(w.value_cache)
    kc2[perm] = w.key_cache
    vc2[perm] = w.value_cache
    w.key_cache, w.value_cache = kc2, vc2
    w.block_tables = perm[w.block_tables.long()].to(torch.int32).contiguous()
    b = gpu_decode(w)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_split_and_unsplit_agree():
    _say("split vs unsplit")
    cfg = _cfg(num_heads=8, num_kv_heads=8, len_args=(700, 1, 333, 1024, 17))
    wh = synth.make_workload(cfg)
    w = to_device(wh)
    gpu_step(w)
    ref = oracle_decode(wh, oracle_caches(wh))
    outs = [gpu_decode(w, p) for p in (16, 64, 512, 2048)]
    torch.cuda.synchronize()
    for p, o in zip((16, 64, 512, 2048), outs):
        assert_close(o, ref, "f16", f"partition {p}")


@pytest.mark.parametrize("name", ["llama7b", "gqa70b", "fp8beams"])
def test_full_size_config(name):
    _say(f"full-size {name}")
    cfg = synth.CONFIGS[name]
    _run_and_check(cfg, what=f"{name} full")


@pytest.mark.parametrize("half", [0, 1])
def test_long_context_every_row(half):
    """The long-context workload at full size (lengths 32K-128K, 512-token partitions merged by the
    long-list merge): every (sequence, head) row of one half of the batch against the oracle, so the
    two cases together check all 8 x 32 rows."""
    cfg = synth.CONFIGS["longctx"]
    seqs = list(range(half * cfg.num_seqs // 2, (half + 1) * cfg.num_seqs // 2))
    _say(f"longctx every row of sequences {seqs}")
    w = synth.make_workload(cfg, device="cuda")
    refs = sequence_reference(cfg, w.tables_np, w.lens_np, w.query.cpu(), w.key_cache, w.value_cache,
                              w.key_new.cpu(), w.value_new.cpu(), seqs)
    out = gpu_step(w)
    got = out.cpu()
    for b in seqs:
        assert_close(got[b], refs[b], cfg.cache_dtype, f"longctx b={b} L={w.lens_np[b]} (all heads)")


@pytest.mark.parametrize("hq,hkv,part", [(4, 4, 0), (16, 2, 0), (4, 4, 32), (16, 2, 64)])
def test_context_lens_clamped_to_the_stated_bounds(hq, hkv, part):
    """Lengths above max_context_len, or above what the page table can hold (16 x its columns), are
    read as the bound; negative lengths as 0 (a zero row).  Compared with the oracle on the clamped
    lengths."""
    _say(f"clamped lengths Hq={hq} Hkv={hkv} part={part}")
    lens = (300, 47, 129, 5, 200, 64)
    cfg = _cfg(name="clamp", num_seqs=len(lens), num_heads=hq, num_kv_heads=hkv, len_args=lens, seed=21,
               partition_size=part)
    wh = synth.make_workload(cfg)
    w = to_device(wh)
    gpu_append(w)
    caches = oracle_caches(wh)
    for cap, cols in ((100, None), (1000, 5)):
        tables = w.block_tables if cols is None else w.block_tables[:, :cols].contiguous()
        bound = cap if cols is None else min(cap, 16 * cols)
        ctx = w.context_lens.clone()
        ctx[3] = -7                                  # negative: an empty sequence
        out = torch.empty_like(w.query)
        pa.pa_decode(out, w.query, w.key_cache, w.value_cache, tables, ctx, cfg.scale, cap, partition_size=part)
        torch.cuda.synchronize()
        eff = np.clip(ctx.cpu().numpy(), 0, bound)
        assert (eff < wh.lens_np).any()
        kc, vc, _, _ = caches
        ref = oracle.paged_decode(synth.bits_np(wh.query), kc, vc, wh.tables_np, eff, cfg.scale, cfg.q_dtype,
                                  cfg.cache_dtype)
        assert_close(out, ref, cfg.cache_dtype, f"clamp cap={cap} cols={cols}")
        assert torch.count_nonzero(out[3]) == 0


@pytest.mark.parametrize("hq,hkv,cd", [(32, 32, "f16"), (32, 8, "fp8_e4m3"), (16, 2, "bf16")])
def test_balanced_split_fewer_ranges_than_teams(hq, hkv, cd):
    """A launch sized for 4096-token contexts over a few short sequences: the grid has all its
    teams (1024 waves, 2048 for FP8; whole groups of eight workgroups, so the waves are
    renumbered per XCD) but the lengths give only a handful of ranges, which go to evenly
    spaced teams while the rest stay idle."""
    _say(f"balanced: fewer ranges than teams Hq={hq} Hkv={hkv} cache={cd}")
    lens = (1, 3, 17, 5, 0, 40)
    cfg = _cfg(name="sparse", num_seqs=len(lens), num_heads=hq, num_kv_heads=hkv, len_args=lens,
               q_dtype="f16" if cd == "f16" else "bf16", cache_dtype=cd, seed=31)
    wh = synth.make_workload(cfg)
    w = to_device(wh)
    gpu_append(w)
    out = torch.empty_like(w.query)
    pa.pa_decode(out, w.query, w.key_cache, w.value_cache, w.block_tables, w.context_lens, cfg.scale, 4096,
                 partition_size=0, k_scale=w.k_scale, v_scale=w.v_scale)
    torch.cuda.synchronize()
    assert_close(out, oracle_decode(wh, oracle_caches(wh)), cd, f"sparse ranges Hq={hq} Hkv={hkv}")


def test_balanced_split_more_than_64_sequences():
    # 130 sequences (lengths walked 64 at a time), some empty, many ranges crossing sequences.
    _say("balanced: 130 sequences, empty ones")
    lens = tuple(int(x) for x in np.random.default_rng(11).integers(0, 400, size=130))
    lens = (0, 0) + lens[2:]
    cfg = _cfg(name="many", num_seqs=130, num_heads=2, num_kv_heads=2, head_dim=64, len_args=lens, seed=12)
    _run_and_check(cfg, partition_size=0)


@pytest.mark.parametrize("hq,hkv,D,part", [(2, 2, 64, 0), (8, 1, 64, 0), (4, 4, 128, 0), (8, 2, 64, 0),
                                           (2, 2, 64, 64)])
def test_512_sequences_mixed_lengths(hq, hkv, D, part):
    """A serving-size batch: 512 sequences, lengths 0..600 (about a tenth empty), so every wave's
    range crosses many sequences and the lookups walk the lengths 64 at a time; VALU (MHA) and
    matrix-core (groups of 8 and 4) paths, balanced split and fixed partitions."""
    _say(f"512 sequences Hq={hq} Hkv={hkv} D={D} part={part}")
    rng = np.random.default_rng(512 + hq + D + part)
    lens = rng.integers(0, 601, size=512)
    lens[rng.random(512) < 0.1] = 0
    cfg = _cfg(name="b512", num_seqs=512, num_heads=hq, num_kv_heads=hkv, head_dim=D, len_args=tuple(int(x) for x in lens),
               q_dtype="bf16", cache_dtype="bf16", seed=14, partition_size=part)
    _run_and_check(cfg, what=f"B=512 G={hq // hkv} part={part}")


@pytest.mark.parametrize("hq,hkv", [(16, 4), (8, 8)])
def test_balanced_split_reused_workspace_repeats_bitwise(hq, hkv):
    _say(f"balanced: reused workspace, repeat bitwise, Hq={hq} Hkv={hkv}")
    lens = (3000, 1, 2047, 0, 1500, 900, 2500, 16)
    cfg = _cfg(name="tiles", num_seqs=len(lens), num_heads=hq, num_kv_heads=hkv, len_args=lens,
               q_dtype="bf16", cache_dtype="bf16", seed=13)
    wh = synth.make_workload(cfg)
    w = to_device(wh)
    ws = pa.alloc_workspace(w.query, hkv, w.max_context_len, 0)
    assert ws is not None
    gpu_step(w)
    outs = []
    for _ in range(3):
        out = torch.empty_like(w.query)
        pa.pa_decode(out, w.query, w.key_cache, w.value_cache, w.block_tables, w.context_lens, cfg.scale,
                     w.max_context_len, partition_size=0, workspace=ws)
        torch.cuda.synchronize()
        outs.append(out)
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))
    assert_close(outs[0], oracle_decode(wh, oracle_caches(wh)), "bf16", "tiles")


def _climbing_keys(wh, span):
    """Rewrite the cached keys and this step's key so that every head's score climbs along its
    context by about ``span`` (natural-log units): K[t] = (t + 1) * step * d + 0.1 * K_random[t],
    with d the unit mean direction of the KV head's query heads.  The running maximum then moves
    at almost every block, which exercises the rescaling of both kernels and the wide range of
    partial maxima that the merge has to fold."""
    cfg = wh.cfg
    B, Hq, Hkv, D = cfg.num_seqs, cfg.num_heads, cfg.num_kv_heads, cfg.head_dim
    G = Hq // Hkv
    q = wh.query.float().view(B, Hkv, G, D)
    d = q.mean(2)
    d = d / d.norm(dim=-1, keepdim=True)
    c = (q * d[:, :, None, :]).sum(-1).mean(-1).clamp(min=0.5) * cfg.scale   # [B, Hkv] score per unit of K along d
    fp8 = cfg.cache_dtype == "fp8_e4m3"
    src = wh.fill_key.float() if fp8 else wh.key_cache.float().view(-1, Hkv, D)
    rows = {int(s): i for i, s in enumerate(wh.fill_slots.tolist())} if fp8 else None
    new_cached = src.clone()
    new_key = wh.key_new.float().clone()
    for b in range(B):
        L = int(wh.lens_np[b])
        if L == 0:
            continue
        step = span / (c[b] * L)                                              # [Hkv]
        for t in range(L):
            slot = int(wh.tables_np[b][t // 16]) * 16 + t % 16
            k = (t + 1) * step[:, None] * d[b]
            if t == L - 1:
                new_key[b] = k + 0.1 * new_key[b]
            else:
                r = rows[slot] if fp8 else slot
                new_cached[r] = k + 0.1 * src[r]
    if fp8:
        wh.fill_key = new_cached.to(wh.fill_key.dtype)
    else:
        wh.key_cache = new_cached.view_as(wh.key_cache).to(wh.key_cache.dtype)
    wh.key_new = new_key.to(wh.key_new.dtype)


@pytest.mark.parametrize("qd,cd,hq,hkv,D,part", [
    ("bf16", "bf16", 8, 1, 128, 0), ("f16", "f16", 4, 1, 64, 0), ("f16", "f16", 2, 2, 128, 0),
    ("bf16", "fp8_e4m3", 8, 2, 128, 0), ("bf16", "bf16", 8, 1, 128, 64), ("f16", "f16", 1, 1, 128, 48)])
def test_scores_climbing_along_the_context(qd, cd, hq, hkv, D, part):
    """Scores that climb by ~200 (natural log) over the context: the softmax reference must move
    many times inside a segment and the partials' maxima differ by up to ~200."""
    _say(f"climbing scores {qd}/{cd} hq={hq} hkv={hkv} D={D} partition={part}")
    cfg = _cfg(q_dtype=qd, cache_dtype=cd, num_heads=hq, num_kv_heads=hkv, head_dim=D,
               len_args=(700, 17, 1, 330, 2100), seed=77)
    wh = synth.make_workload(cfg)
    _climbing_keys(wh, 200.0)
    w = to_device(wh)
    out = gpu_step(w, part)
    ref = oracle_decode(wh, oracle_caches(wh))
    assert_close(out, ref, cd, f"climbing {qd}/{cd} {hq}/{hkv}")
