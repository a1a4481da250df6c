"""GPU parity of shared-prefix paged decode (pa_decode_shared_prefix) against the float64 oracle.

Sequences of one group share their first page-table entries (beam search and parallel
sampling share prefix blocks through reference counts); the method's result is still
plain paged attention of every sequence over its own tokens, so the reference is the
oracle's paged_decode on the same tables.  Every slot no sequence reads holds NaN
(FP8: the NaN code and NaN scales), so a block read for the wrong sequence or past a
sequence's length shows up in the output.
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

TDT = {"f16": torch.float16, "bf16": torch.bfloat16}


def _say(msg):
    print(f"[case] {msg}", flush=True)


def _group_lens(kind, S, rng):
    """(shared blocks, prefix_blocks claim, lengths) of one group."""
    if kind == "prefix":            # shared prefix, ragged private parts, one ends at the prefix
        P = int(rng.integers(2, 9))
        lens = [P * 16 + int(rng.integers(1, 120)) for _ in range(S)]
        lens[-1] = P * 16
        return P, P, lens
    if kind == "none":              # no sharing
        return 0, 0, [int(rng.integers(1, 300)) for _ in range(S)]
    if kind == "inside":            # every sequence ends inside the shared blocks; the claim is clamped
        P = int(rng.integers(2, 6))
        return P, 999, [int(rng.integers(1, P * 16 + 1)) for _ in range(S)]
    if kind == "empty_member":      # one empty sequence: nothing is shared
        P = 3
        lens = [P * 16 + int(rng.integers(0, 50)) for _ in range(S)]
        lens[0] = 0
        return P, P, lens
    if kind == "all_empty":
        return 0, 2, [0] * S
    if kind == "long":
        P = int(rng.integers(30, 50))
        return P, P, [P * 16 + int(rng.integers(1, 400)) for _ in range(S)]
    raise ValueError(kind)


def _case(S, hq, hkv, D, qd, cd, kinds, seed):
    """Pools, tables, lengths and queries for groups of S sequences described by ``kinds``."""
    rng = np.random.default_rng(seed)
    specs = [_group_lens(k, S, rng) for k in kinds]
    lens = [L for _, _, ls in specs for L in ls]
    B = len(lens)
    nblk = [(L + 15) // 16 for L in lens]
    max_blocks = max(1, max(nblk))
    need = sum(P + sum(max(0, n - P) for n in (nblk[g * S:(g + 1) * S])) for g, (P, _, _) in enumerate(specs))
    num_blocks = need + 8
    ids = rng.permutation(num_blocks)
    nxt = 0
    tables = np.full((B, max_blocks), num_blocks - 1, dtype=np.int32)   # padding: a never-read block
    for g, (P, _, _) in enumerate(specs):
        shared = ids[nxt:nxt + P]
        nxt += P
        for s in range(S):
            b = g * S + s
            tables[b, :min(P, nblk[b])] = shared[:min(P, nblk[b])]
            for j in range(P, nblk[b]):
                tables[b, j] = ids[nxt]
                nxt += 1
    assert nxt <= num_blocks - 8
    read = np.zeros((num_blocks, 16), dtype=bool)
    for b in range(B):
        for t in range(lens[b]):
            read[tables[b, t // 16], t % 16] = True

    g = torch.Generator().manual_seed(seed)
    shape = (num_blocks, 16, hkv, D)
    if cd == "fp8_e4m3":
        def codes():   # sign, exponent field 0..8, mantissa: magnitudes below 4, no NaN code
            sign = torch.randint(0, 2, shape, generator=g, dtype=torch.int32)
            exp = torch.randint(0, 9, shape, generator=g, dtype=torch.int32)
            man = torch.randint(0, 8, shape, generator=g, dtype=torch.int32)
            return (sign << 7 | exp << 3 | man).to(torch.uint8)
        kc, vc = codes(), codes()
        ks = (0.25 + 0.25 * torch.rand(num_blocks, 16, generator=g)).float()
        vs = (0.25 + 0.25 * torch.rand(num_blocks, 16, generator=g)).float()
        mask = torch.from_numpy(~read)
        kc[mask] = 0x7F
        vc[mask] = 0x7F
        ks[mask] = float("nan")
        vs[mask] = float("nan")
    else:
        kc = torch.randn(shape, generator=g).to(TDT[cd])
        vc = torch.randn(shape, generator=g).to(TDT[cd])
        mask = torch.from_numpy(~read)
        kc[mask] = float("nan")
        vc[mask] = float("nan")
        ks = vs = None
    q = torch.randn(B, hq, D, generator=g).to(TDT[qd])
    prefix = np.array([claim for _, claim, _ in specs], dtype=np.int32)
    return dict(q=q, kc=kc, vc=vc, ks=ks, vs=vs, tables=tables, lens=np.array(lens, dtype=np.int32),
                prefix=prefix, S=S, qd=qd, cd=cd, scale=1.0 / np.sqrt(D), max_len=max(1, max(lens)))


def _reference(c):
    return oracle.paged_decode(bits_np(c["q"]), bits_np(c["kc"]), bits_np(c["vc"]), c["tables"], c["lens"],
                               c["scale"], c["qd"], c["cd"],
                               None if c["ks"] is None else c["ks"].numpy(),
                               None if c["vs"] is None else c["vs"].numpy())


def _gpu(c, workspace=None):
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in c.items()}
    tables = torch.from_numpy(c["tables"]).cuda()
    lens = torch.from_numpy(c["lens"]).cuda()
    prefix = torch.from_numpy(c["prefix"]).cuda()
    out = torch.empty_like(d["q"])
    pa.pa_decode_shared_prefix(out, d["q"], d["kc"], d["vc"], tables, lens, prefix, c["S"], c["scale"],
                               c["max_len"], k_scale=d["ks"], v_scale=d["vs"], workspace=workspace)
    plain = torch.empty_like(d["q"])
    pa.pa_decode(plain, d["q"], d["kc"], d["vc"], tables, lens, c["scale"], c["max_len"], k_scale=d["ks"],
                 v_scale=d["vs"])
    torch.cuda.synchronize()
    return out, plain


KINDS = ["prefix", "none", "inside", "empty_member", "all_empty", "long", "prefix"]


@pytest.mark.parametrize("S,hq,hkv,D,qd,cd", [
    (4, 32, 8, 128, "bf16", "bf16"),        # 4 beams x 4 heads: full 16-row tiles
    (2, 64, 8, 128, "bf16", "bf16"),        # GQA group 8: two sequences per tile
    (4, 32, 8, 128, "bf16", "fp8_e4m3"),
    (2, 8, 8, 64, "f16", "f16"),            # MHA: one head per sequence
    (16, 16, 16, 64, "f16", "f16"),         # 16 sequences of one head
    (3, 15, 3, 128, "f16", "fp8_e4m3"),     # group 5 x 3 sequences = 15 rows
    (1, 16, 1, 128, "bf16", "bf16"),        # one sequence per group, group of 16 heads
])
def test_shared_prefix_sweep(S, hq, hkv, D, qd, cd):
    _say(f"shared prefix S={S} Hq={hq} Hkv={hkv} D={D} q={qd} cache={cd}")
    c = _case(S, hq, hkv, D, qd, cd, KINDS, seed=100 + S * 7 + hq)
    ref = _reference(c)
    out, plain = _gpu(c)
    tol = "fp8_e4m3" if cd == "fp8_e4m3" else qd
    assert_close(out, ref, tol, f"shared prefix S={S} G={hq // hkv}")
    assert_close(plain, ref, tol, f"pa_decode on the same tables S={S} G={hq // hkv}")
    empty = c["lens"] == 0
    assert torch.all(out.cpu()[torch.from_numpy(empty)] == 0)


def test_shared_prefix_repeat_is_bitwise_deterministic():
    _say("shared prefix: two calls, one workspace, bitwise equal")
    c = _case(4, 32, 8, 128, "bf16", "bf16", ["long", "prefix", "long", "none"], seed=7)
    ws = torch.empty(pa.shared_prefix_workspace_bytes(16, 4, 32, 8, 128, c["max_len"]), dtype=torch.uint8,
                     device="cuda")
    a, _ = _gpu(c, ws)
    b, _ = _gpu(c, ws)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_fp8_beams_full_size():
    # 16 prompts x 4 beams, 1024-token prefix (64 blocks) shared by the beams, FP8 cache
    # written by the device append (every cached token, then this step's new tokens).
    _say("fp8beams full size through pa_decode_shared_prefix")
    cfg = synth.CONFIGS["fp8beams"]
    wh = synth.make_workload(cfg)
    kc, vc, ks, vs = oracle_caches(wh)
    ref = oracle.paged_decode(bits_np(wh.query), kc, vc, wh.tables_np, wh.lens_np, cfg.scale, cfg.q_dtype,
                              cfg.cache_dtype, ks, vs)
    w = to_device(wh)
    gpu_append(w)
    groups = cfg.num_seqs // cfg.beams
    prefix = torch.full((groups,), cfg.prefix_len // 16, dtype=torch.int32, device="cuda")
    out = torch.empty_like(w.query)
    pa.pa_decode_shared_prefix(out, w.query, w.key_cache, w.value_cache, w.block_tables, w.context_lens, prefix,
                               cfg.beams, cfg.scale, w.max_context_len, k_scale=w.k_scale, v_scale=w.v_scale)
    torch.cuda.synchronize()
    assert_close(out, ref, cfg.cache_dtype, "fp8beams shared prefix")


def test_shared_prefix_rejects_bad_groups():
    _say("shared prefix: group sizes that do not divide the batch or overflow a tile")
    c = _case(2, 16, 2, 64, "f16", "f16", ["prefix", "none"], seed=3)     # 4 sequences, group of 8 heads
    q, kc, vc = c["q"].cuda(), c["kc"].cuda(), c["vc"].cuda()
    tables = torch.from_numpy(c["tables"]).cuda()
    lens = torch.from_numpy(c["lens"]).cuda()
    out = torch.empty_like(q)
    one = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):          # 4 sequences in groups of 3
        pa.pa_decode_shared_prefix(out, q, kc, vc, tables, lens, one, 3, c["scale"], c["max_len"])
    with pytest.raises(pa.PagedAttnError):   # 4 sequences x 8 heads = 32 rows > 16
        pa.pa_decode_shared_prefix(out, q, kc, vc, tables, lens, one, 4, c["scale"], c["max_len"])


def test_shared_prefix_more_than_64_groups():
    # 70 groups of 2 sequences: the balanced split walks the groups 64 at a time.
    _say("shared prefix: 70 groups (group table walked 64 at a time)")
    kinds = (["prefix", "none", "inside", "long", "empty_member", "all_empty", "prefix"] * 10)[:70]
    c = _case(2, 16, 4, 64, "f16", "f16", kinds, seed=91)
    ref = _reference(c)
    out, plain = _gpu(c)
    assert_close(out, ref, "f16", "shared prefix, 70 groups")
    assert_close(plain, ref, "f16", "pa_decode on the same tables, 140 sequences")
