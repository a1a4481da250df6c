"""Benchmark: one decode step of paged attention on one MI355X.

A step is the whole hot path over one batch: the slot-mapped append of each
sequence's new token, then paged decode attention over every sequence's cache
(split over partitions and merged when a sequence is longer than one
partition).  The default workload is the LLaMA-7B-shaped single layer: B=32
sequences, 32 query / 32 KV heads, head_dim 128, f16 cache, 16-token blocks,
context lengths uniform in [1, 2048], pool = blocks in use + 10 %, physical
blocks in seeded random order.  Inputs are synthetic (seeded N(0,1)).

Timing: W untimed steps, then K timed steps between two device
synchronisations; each step uses the next of R pool replicas (R * pool bytes
well above the 256 MB Infinity Cache), so the KV bytes come from HBM.  Kernels
are launched from Python on torch's current stream (--graphs replays captured
HIP graphs of the same launches instead).  One pair of HIP events on the launch
stream brackets the K timed steps: the GPU time of one call for the roofline
line (the default step is one pa_decode_append call).  A separate, shorter pass
with events around every call gives the spread of one call's duration.

Prints one JSON line.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode attention: tokens/s and effective HBM GB/s (% of peak), 1×MI355X"
HBM_PEAK_GBS = 8000.0

WORKLOAD_TEXT = {
    "llama7b": "LLaMA-7B-shaped single-layer paged decode: B=32, Hq=Hkv=32, D=128, f16 KV/Q, fp32 accumulate, "
               "16-token blocks, context lens U[1,2048], pool +10%, permuted blocks",
    "gqa70b": "GQA 70B-shaped single layer: B=64, Hq=64, Hkv=8, D=128, bf16, 16-token blocks, context lens "
              "lognormal (median 1024, sigma 1, clip [16,4096]), pool +10%, permuted blocks",
    "longctx": "long-context split-K decode: B=8, Hq=Hkv=32, D=128, f16, context lens U[32768,131072], "
               "512-token partitions",
    "fp8beams": "fp8-e4m3 KV with per-token scales, 16 prompts x 4 beams sharing 1024-token prefixes + 256 "
                "private tokens, Hq=32, Hkv=8, D=128, Q bf16",
    "tiny": "tiny paged decode: B=4, lens {1,17,33,50}, Hq=Hkv=4, D=64, f16",
    "llama7b_b256": "LLaMA-7B-shaped single-layer paged decode at B=256: Hq=Hkv=32, D=128, f16, context lens "
                    "U[1,2048], pool +10%, permuted blocks",
}


def algorithmic_bytes(w, window=0):
    """Bytes the method must read per decode: KV rows + scales, Q, page-table entries, lengths.

    With a sliding window only the last `window` tokens of each sequence (and the table entries
    of their blocks) count.
    """
    import numpy as np
    cfg = w.cfg
    eb = 1 if cfg.cache_dtype == "fp8_e4m3" else 2
    lens = w.lens_np.astype(np.int64)
    if window > 0:
        first = np.maximum(lens - window, 0)
        kv_tokens = int(np.sum(lens - first))
        blocks = int(np.sum((lens + 15) // 16 - first // 16))
        return (kv_tokens * cfg.num_kv_heads * cfg.head_dim * 2 * eb + (kv_tokens * 8 if eb == 1 else 0)
                + cfg.num_seqs * cfg.num_heads * cfg.head_dim * 2 + blocks * 4 + cfg.num_seqs * 4)
    if cfg.beams > 1:
        # unique bytes: shared prefix blocks counted once
        prompts = cfg.num_seqs // cfg.beams
        tokens = prompts * cfg.prefix_len + int(np.sum(lens - cfg.prefix_len))
    else:
        tokens = int(lens.sum())
    kv = tokens * cfg.num_kv_heads * cfg.head_dim * 2 * eb
    if eb == 1:
        kv += tokens * 8
    q = cfg.num_seqs * cfg.num_heads * cfg.head_dim * 2
    table = int(np.sum((lens + 15) // 16)) * 4 + cfg.num_seqs * 4
    return kv + q + table


def measured_traffic(workload):
    """HBM bytes per decode call from the committed FETCH_SIZE / WRITE_SIZE summary, or None.

    profiles/decode_traffic_<workload>.txt records the counter-derived bytes (scaled by the
    plain-copy calibration) together with a SHA-256 of the kernel sources it was taken with;
    the figure is only reported while those sources are unchanged.
    """
    import hashlib
    path = os.path.join(ROOT, "profiles", f"decode_traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path, encoding="utf-8"):
        if ":" in line and line.split(":", 1)[0] in ("traffic_bytes_per_call", "kernel_sources",
                                                      "kernel_sources_sha256"):
            k, v = line.split(":", 1)
            fields[k] = v.strip()
    if len(fields) != 3:
        return None
    h = hashlib.sha256()
    for src in fields["kernel_sources"].split():
        try:
            h.update(open(os.path.join(ROOT, src), "rb").read())
        except OSError:
            return None
    return int(fields["traffic_bytes_per_call"]) if h.hexdigest() == fields["kernel_sources_sha256"] else None


def append_bytes(w):
    """Bytes the append of a step moves: the new K/V rows read (query dtype) and written into the
    cache (plus one scale per token and pool for FP8)."""
    cfg = w.cfg
    eb = 1 if cfg.cache_dtype == "fp8_e4m3" else 2
    rows = cfg.num_seqs * cfg.num_kv_heads * cfg.head_dim
    return 2 * rows * 2 + 2 * rows * eb + (2 * 4 * cfg.num_seqs if eb == 1 else 0)


def time_workload(name, steps, warmup, replicas, sample=None, partition_size=None, use_graphs=False, window=0,
                  q_len=1, shared_prefix=False, fused=False):
    import torch
    import paged_kv_cache_187_amd as pa
    import synth

    overrides = {} if partition_size is None else {"partition_size": partition_size}
    w = synth.make_workload(name, device="cuda", **overrides)
    cfg = w.cfg
    # pre-step host copies for the CPU baseline (sample = heads kept per sequence, 0 = all)
    host = None if sample is None else cpu_sample(w, heads_per_seq=sample or None)
    kcs = [w.key_cache] + [w.key_cache.clone() for _ in range(replicas - 1)]
    vcs = [w.value_cache] + [w.value_cache.clone() for _ in range(replicas - 1)]
    kss = [w.k_scale] + [None if w.k_scale is None else w.k_scale.clone() for _ in range(replicas - 1)]
    vss = [w.v_scale] + [None if w.v_scale is None else w.v_scale.clone() for _ in range(replicas - 1)]
    if w.fill_slots is not None:
        for r in range(replicas):
            pa.pa_append_kv(w.fill_key, w.fill_value, kcs[r], vcs[r], w.fill_slots, kss[r], vss[r])
    part = cfg.partition_size
    max_len = w.max_context_len
    if q_len > 1:   # q_len new tokens per sequence: its last q_len cached positions
        query = torch.randn(cfg.num_seqs, q_len, cfg.num_heads, cfg.head_dim, device="cuda").to(w.query.dtype)
        n = pa.load_library().pa_decode_multi_workspace_bytes(cfg.num_seqs, q_len, cfg.num_heads, cfg.num_kv_heads,
                                                             cfg.head_dim, max_len, part)
        ws = torch.empty(n, dtype=torch.uint8, device="cuda") if n else None
    elif shared_prefix:   # the beams of one prompt form a group sharing its prefix blocks
        query = w.query
        prefix = torch.full((cfg.num_seqs // cfg.beams,), cfg.prefix_len // 16, dtype=torch.int32, device="cuda")
        n = pa.shared_prefix_workspace_bytes(cfg.num_seqs, cfg.beams, cfg.num_heads, cfg.num_kv_heads, cfg.head_dim,
                                             max_len)
        ws = torch.empty(n, dtype=torch.uint8, device="cuda") if n else None
    else:
        query = w.query
        ws = pa.alloc_workspace(w.query, cfg.num_kv_heads, w.max_context_len, part)
    out = torch.empty_like(query)

    assert not (fused and (q_len > 1 or shared_prefix or window > 0)), "the fused step is the plain decode"

    def append(r):
        if not fused:   # the fused step appends inside the decode call
            pa.pa_append_kv(w.key_new, w.value_new, kcs[r], vcs[r], w.slot_mapping, kss[r], vss[r])

    def decode(r):
        if fused:
            pa.pa_decode_append(out, w.query, w.key_new, w.value_new, kcs[r], vcs[r], w.block_tables,
                                w.context_lens, cfg.scale, max_len, partition_size=part, k_scale=kss[r],
                                v_scale=vss[r], workspace=ws)
        elif q_len > 1:
            pa.pa_decode_multi(out, query, kcs[r], vcs[r], w.block_tables, w.context_lens, cfg.scale, max_len,
                               partition_size=part, k_scale=kss[r], v_scale=vss[r], workspace=ws)
        elif shared_prefix:
            pa.pa_decode_shared_prefix(out, w.query, kcs[r], vcs[r], w.block_tables, w.context_lens, prefix,
                                       cfg.beams, cfg.scale, max_len, k_scale=kss[r], v_scale=vss[r], workspace=ws)
        elif window > 0:
            pa.pa_decode_sliding(out, w.query, kcs[r], vcs[r], w.block_tables, w.context_lens, cfg.scale, max_len,
                                 window, partition_size=part, k_scale=kss[r], v_scale=vss[r], workspace=ws)
        else:
            pa.pa_decode(out, w.query, kcs[r], vcs[r], w.block_tables, w.context_lens, cfg.scale, max_len,
                         partition_size=part, k_scale=kss[r], v_scale=vss[r], workspace=ws)

    for i in range(warmup):
        append(i % replicas)
        decode(i % replicas)
    torch.cuda.synchronize()
    if use_graphs:
        # One HIP graph per replica for the append and one for the decode: replaying them keeps
        # the host from pacing the GPU, and the decode replay stays separately timeable.
        graphs = []
        for r in range(replicas):
            ga, gd = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
            with torch.cuda.graph(ga):
                append(r)
            with torch.cuda.graph(gd):
                decode(r)
            graphs.append((ga, gd))
        run_append = lambda r: graphs[r][0].replay()
        run_decode = lambda r: graphs[r][1].replay()
        for i in range(warmup):
            run_append(i % replicas)
            run_decode(i % replicas)
    else:
        run_append, run_decode = append, decode
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    # Timed region: `steps` whole steps with one event pair around all of them on the launch
    # stream (events around every call put their own packets between the steps and slow each
    # step by several microseconds).
    region = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    region[0].record(stream)
    for i in range(steps):
        r = (warmup + i) % replicas
        run_append(r)
        run_decode(r)
    region[1].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    step_gpu_ms = region[0].elapsed_time(region[1]) / steps
    # A separate pass with events around each decode call: the spread of one call's duration,
    # and for a step of two calls the decode call alone.
    n_ev = min(steps, 60)
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_ev)]
    for i in range(n_ev):
        r = (warmup + steps + i) % replicas
        run_append(r)
        events[i][0].record(stream)
        run_decode(r)
        events[i][1].record(stream)
    torch.cuda.synchronize()
    dec_ms = sorted(e[0].elapsed_time(e[1]) for e in events)
    n = len(dec_ms)
    kind = ("fused" if fused else f"q_len {q_len}" if q_len > 1 else "shared prefix" if shared_prefix
            else f"window {window}" if window > 0 else "append + decode")
    print(f"[bench] {name} ({kind}): {step_gpu_ms * 1e3:.1f} us per step", file=sys.stderr, flush=True)
    return {
        "w": w,
        "cpu_sample": host,
        "ms_per_step": (t1 - t0) * 1e3 / steps,
        "step_gpu_ms": step_gpu_ms,
        # the fused step is one call: its duration is the region's; otherwise the per-call events'
        "decode_ms_mean": step_gpu_ms if fused else sum(dec_ms) / n,
        "decode_timing": ("events around the timed steps (the step is the call)" if fused
                          else "events around each decode call (separate pass)"),
        "decode_ms_p10": dec_ms[n // 10],
        "decode_ms_p50": dec_ms[n // 2],
        "decode_ms_p90": dec_ms[min(n - 1, (9 * n) // 10)],
        "partition_size": pa.decode_partition_size(cfg.num_seqs, cfg.num_heads, cfg.num_kv_heads, cfg.head_dim,
                                                   max_len, part),
        "bytes": algorithmic_bytes(w, window) + (q_len - 1) * cfg.num_seqs * cfg.num_heads * cfg.head_dim * 2
                 + (append_bytes(w) if fused else 0),
        "q_len": q_len,
        "fused": fused,
    }


def unique_blocks(name):
    """Physical blocks holding the cached tokens of workload `name` (shared prefix blocks once),
    from the same seeded draws as synth.make_workload, without building the pools."""
    import numpy as np
    from synth import workloads as W
    cfg = W.CONFIGS[name]
    rng = np.random.default_rng(cfg.seed)
    lens = W.sample_lengths(cfg, rng)
    return W.build_tables(cfg, lens, rng)[2]


def read_ceiling(steps=50, warmup=5):
    """Achievable read bandwidth on this GPU, reported beside (not as) the decode figures.

    stream: a plain streaming read of a 2 GiB buffer.  paged_gather: the llama7b decode's
    access pattern without the attention (every head's 256-byte rows of 16-token blocks of 32
    KV heads, blocks in random order, next block's loads in flight) in the decode's order
    (teams of one wave per KV head reading the same blocks; 1024 waves, the decode's count),
    4400 blocks (577 MB) per launch; paged_gather_head_major: the same rows
    with each wave reading one head of consecutive blocks (2048 waves).
    paged_gather_by_workload: the team-order probe in the geometry of the gqa70b (8 KV heads,
    256-byte rows) and fp8beams (8 KV heads, 128-byte rows of one-byte codes) workloads at 1024
    waves, over as many block reads as the workload's K and V pools hold unique
    blocks (the FP8 scales aside).  Each launch takes its blocks from one of three disjoint
    sets of a 2 GiB pool.  Probe kernels of libpaprobe.so
    (paged_kv_cache_187_amd/probe/pa_probe.hip), timed as the decode step is: one HIP event
    pair around `steps` back-to-back launches.
    """
    import ctypes
    import torch
    from paged_kv_cache_187_amd.build import PROBE_PATH
    lib = ctypes.CDLL(PROBE_PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.pa_probe_stream.argtypes = [vp, i64, vp, i32, vp]
    lib.pa_probe_gather.argtypes = [vp, vp, i32, i32, i32, i64, i32, vp, vp]
    lib.pa_probe_gather_teams.argtypes = [vp, vp, i32, i32, i32, i64, i32, vp, vp]
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    nbytes = 2 << 30
    buf = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    blocks = 4096
    sink = torch.empty(max(blocks * 256, 2048 * 64), dtype=torch.int32, device="cuda")
    g = torch.Generator().manual_seed(7)

    def run(launch, n):
        # timed like the decode step: one event pair around n back-to-back launches (events
        # between launches would add their own packets to every launch)
        for i in range(warmup):
            assert launch(i) == 0
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(n):
            assert launch(warmup + i) == 0
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e-3 / n

    def gather(hkv, row, n_ids, waves, teams=True):
        blk = 16 * hkv * row
        num_blocks = nbytes // blk
        assert 3 * n_ids <= num_blocks and waves * 64 <= sink.numel()
        perm = torch.randperm(num_blocks, generator=g)[:3 * n_ids].to(torch.int32).cuda()
        id_sets = [perm[i * n_ids:(i + 1) * n_ids].contiguous() for i in range(3)]
        probe = lib.pa_probe_gather_teams if teams else lib.pa_probe_gather
        t = run(lambda i: probe(buf.data_ptr(), id_sets[i % 3].data_ptr(), n_ids, hkv, row, num_blocks, waves,
                                sink.data_ptr(), sp), steps)
        gathered = n_ids * blk
        order = "teams of one wave per KV head on the same blocks" if teams else "one head per wave, head-major"
        return {"bytes": gathered, "GBs": round(gathered / t / 1e9, 1),
                "frac_of_peak": round(gathered / t / 1e9 / HBM_PEAK_GBS, 4),
                "pattern": f"{row}-byte head rows of random 16-token blocks, {hkv} KV heads, {n_ids} block reads, "
                           f"{waves} waves, {order}"}

    t_stream = run(lambda i: lib.pa_probe_stream(buf.data_ptr(), nbytes, sink.data_ptr(), blocks, sp), steps)
    res = {"stream_read": {"bytes": nbytes, "GBs": round(nbytes / t_stream / 1e9, 1),
                           "frac_of_peak": round(nbytes / t_stream / 1e9 / HBM_PEAK_GBS, 4)},
           "paged_gather": gather(32, 256, 4400, 1024),
           "paged_gather_head_major": gather(32, 256, 4400, 2048, teams=False),
           "paged_gather_by_workload": {"gqa70b": gather(8, 256, 2 * unique_blocks("gqa70b"), 1024),
                                        "fp8beams": gather(8, 128, 2 * unique_blocks("fp8beams"), 1024)}}
    del buf
    torch.cuda.empty_cache()
    return res


def time_copy_blocks(steps, warmup, pairs, num_blocks=4096, replicas=2):
    """pa_copy_blocks on llama7b-shaped blocks (32 KV heads x 128 x f16: 128 KiB per pool per block).

    `pairs` random (src, dst) pairs with distinct destinations that are never sources; bytes moved
    per call = pairs x 2 pools x 128 KiB, read once and written once.  Pools of `num_blocks` blocks
    (1 GiB for both pools at 4096) alternate between calls so the data comes from HBM.
    """
    import numpy as np
    import torch
    import paged_kv_cache_187_amd as pa

    hkv, d = 32, 128
    block_bytes = 16 * hkv * d * 2
    pools = []
    for r in range(replicas):
        pools.append((torch.empty(num_blocks, 16, hkv, d, dtype=torch.float16, device="cuda").normal_(),
                      torch.empty(num_blocks, 16, hkv, d, dtype=torch.float16, device="cuda").normal_()))
    ids = np.random.default_rng(5).permutation(num_blocks)
    mapping = torch.from_numpy(np.stack([ids[:pairs], ids[pairs:2 * pairs]], 1).astype(np.int64)).cuda()
    for i in range(warmup):
        pa.pa_copy_blocks(*pools[i % replicas], mapping)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i, (a, b) in enumerate(ev):
        a.record(stream)
        pa.pa_copy_blocks(*pools[i % replicas], mapping)
        b.record(stream)
    torch.cuda.synchronize()
    us = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)
    mean = sum(us) / len(us)
    moved = pairs * 2 * block_bytes * 2
    return {"pairs": pairs, "block_bytes_per_pool": block_bytes, "bytes_moved": moved,
            "us_mean": round(mean, 2), "us_p10_p50_p90": [round(us[len(us) // 10], 2), round(us[len(us) // 2], 2),
                                                          round(us[(9 * len(us)) // 10], 2)],
            "effective_GBs": round(moved / (mean * 1e-6) / 1e9, 1),
            "frac_of_peak": round(moved / (mean * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}


def time_swap(steps, warmup, pairs=256, num_blocks=1024):
    """pa_swap_blocks between a GPU pool and a pinned host pool, llama7b-shaped blocks.

    Swap-out copies `pairs` random GPU blocks (K and V, 128 KiB each) to the host pool and swap-in
    copies them back to other GPU blocks; bytes moved per call = pairs x 2 x 128 KiB over PCIe.
    """
    import numpy as np
    import torch
    import paged_kv_cache_187_amd as pa

    hkv, d = 32, 128
    gpu = (torch.empty(num_blocks, 16, hkv, d, dtype=torch.float16, device="cuda").normal_(),
           torch.empty(num_blocks, 16, hkv, d, dtype=torch.float16, device="cuda").normal_(), None, None)
    host = (torch.zeros(pairs, 16, hkv, d, dtype=torch.float16, pin_memory=True),
            torch.zeros(pairs, 16, hkv, d, dtype=torch.float16, pin_memory=True), None, None)
    ids = np.random.default_rng(6).permutation(num_blocks)
    out_map = torch.from_numpy(np.stack([ids[:pairs], np.arange(pairs)], 1).astype(np.int64)).cuda()
    in_map = torch.from_numpy(np.stack([np.arange(pairs), ids[pairs:2 * pairs]], 1).astype(np.int64)).cuda()
    moved = pairs * 2 * 16 * hkv * d * 2
    res = {"pairs": pairs, "bytes_per_call": moved}
    stream = torch.cuda.current_stream()
    for name, src, dst, m in (("swap_out", gpu, host, out_map), ("swap_in", host, gpu, in_map)):
        for _ in range(warmup):
            pa.pa_swap_blocks(src, dst, m)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for a, b in ev:
            a.record(stream)
            pa.pa_swap_blocks(src, dst, m)
            b.record(stream)
        torch.cuda.synchronize()
        us = sum(a.elapsed_time(b) for a, b in ev) * 1e3 / steps
        res[name] = {"us_mean": round(us, 1), "GBs": round(moved / (us * 1e-6) / 1e9, 1)}
    return res


# ---------------------------------------------------------------------------
# CPU baseline: the float64 oracle, unchanged, on the host's cores.  A pool of worker
# processes (one BLAS thread each) is started before anything touches the GPU; each worker
# gets a share of a workload's sequences as compact host copies of their pre-step caches and
# times whole oracle steps on them (the append of the sequence's new token, then the decode of
# its rows).  Nothing the HIP path writes reaches the oracle.

def _oracle_worker_init():
    from threadpoolctl import threadpool_limits
    global _BLAS_LIMIT
    _BLAS_LIMIT = threadpool_limits(limits=1)   # kept alive: one BLAS thread per worker


def _oracle_worker_ready(_):
    import numpy as np  # noqa: F401
    import oracle  # noqa: F401
    return os.getpid()


def _oracle_step_chunk(chunk, budget_s):
    """Times oracle steps over ``chunk`` (a list of per-sequence samples) for about ``budget_s``.

    Untimed set-up: an FP8 sample's cached tokens are first quantised into its compact pool by
    the oracle's own quantising append.  Timed: repetitions of, for every sample, the append of
    the new token followed by the decode of the sample's rows.  Returns (seconds, repetitions).
    """
    import numpy as np
    import oracle

    prepared = []
    for smp in chunk:
        L, nblk = smp["L"], smp["nblk"]
        if smp["cache_dtype"] == "fp8_e4m3":
            hkv, d = smp["kn"].shape[1:]
            kc = np.full((nblk, 16, hkv, d), 0x7F, dtype=np.uint8)
            ks = np.full((nblk, 16), np.nan, dtype=np.float32)
            kc, vc, ks, vs = oracle.append_kv_e4m3(kc, kc.copy(), ks, ks.copy(), smp["fill_k"], smp["fill_v"],
                                                   smp["src_dtype"], np.arange(L - 1, dtype=np.int64))
            prepared.append((smp, kc, vc, ks, vs))
        else:
            prepared.append((smp, smp["kc"], smp["vc"], None, None))

    def one_rep():
        for smp, kc, vc, ks, vs in prepared:
            L, nblk = smp["L"], smp["nblk"]
            slot = np.array([L - 1], dtype=np.int64)
            if ks is not None:
                k2, v2, ks2, vs2 = oracle.append_kv_e4m3(kc, vc, ks, vs, smp["kn"], smp["vn"], smp["src_dtype"], slot)
            else:
                (k2, v2), ks2, vs2 = oracle.append_kv(kc, vc, smp["kn"], smp["vn"], slot), None, None
            out = oracle.paged_decode(smp["q"][None], k2, v2, np.arange(nblk)[None, :], np.array([L]), smp["scale"],
                                      smp["q_dtype"], smp["cache_dtype"], ks2, vs2)
            assert np.all(np.isfinite(out))

    t0 = time.perf_counter()
    one_rep()
    t1 = time.perf_counter() - t0
    reps = 1 + max(0, min(10000, int(budget_s / max(t1, 1e-6)) - 1))
    for _ in range(reps - 1):
        one_rep()
    return time.perf_counter() - t0, reps


def start_oracle_pool():
    """Worker processes for the CPU baseline, started (spawn) before the GPU is touched, so that no
    process is ever started from one that has initialised the GPU.  Sized to the host cores this
    process may run on, at most 16 (one GPU's share of a host)."""
    import concurrent.futures as cf
    import multiprocessing as mp
    cores = len(os.sched_getaffinity(0))
    workers = max(1, min(16, cores))
    pool = cf.ProcessPoolExecutor(max_workers=workers, mp_context=mp.get_context("spawn"),
                                  initializer=_oracle_worker_init)
    pids = set(pool.map(_oracle_worker_ready, range(4 * workers)))
    return pool, workers, cores, len(pids)


def cpu_sample(w, heads_per_seq=None, seed=0):
    """Host copies of what the oracle needs for each sequence of workload ``w``, taken before the
    step's append: the sequence's blocks (compact, in logical order), its queries, its new token,
    and for an FP8 cache the source values of its cached tokens.  ``heads_per_seq``: keep only
    that many seeded query heads (and their KV heads) per sequence (16-bit caches)."""
    import numpy as np
    import torch
    from synth import bits_np
    cfg = w.cfg
    g = cfg.num_heads // cfg.num_kv_heads
    rng = np.random.default_rng(seed)
    fp8 = cfg.cache_dtype == "fp8_e4m3"
    fill_row = {}
    if fp8:
        fill_row = {int(s): i for i, s in enumerate(w.fill_slots.cpu().tolist())}
        fk, fv = w.fill_key.cpu(), w.fill_value.cpu()
    q_all = w.query.cpu()
    kn_all, vn_all = w.key_new.cpu(), w.value_new.cpu()
    samples = []
    for b in range(cfg.num_seqs):
        L = int(w.lens_np[b])
        if L == 0:
            continue
        nblk = (L + 15) // 16
        if heads_per_seq is None:
            heads = list(range(cfg.num_heads))
            kv = list(range(cfg.num_kv_heads))
        else:
            assert not fp8 and g == 1, "head sampling is for MHA 16-bit caches"
            heads = sorted(int(h) for h in rng.choice(cfg.num_heads, size=heads_per_seq, replace=False))
            kv = heads
        smp = {"L": L, "nblk": nblk, "scale": cfg.scale, "q_dtype": cfg.q_dtype, "cache_dtype": cfg.cache_dtype,
               "src_dtype": cfg.src_dtype, "heads": len(heads), "all_heads": cfg.num_heads,
               "q": bits_np(q_all[b, heads]), "kn": bits_np(kn_all[b:b + 1, kv]), "vn": bits_np(vn_all[b:b + 1, kv])}
        if fp8:
            rows = [fill_row[int(w.tables_np[b][t // 16]) * 16 + t % 16] for t in range(L - 1)]
            idx = torch.tensor(rows, dtype=torch.int64)
            smp["fill_k"], smp["fill_v"] = bits_np(fk.index_select(0, idx)), bits_np(fv.index_select(0, idx))
        else:
            ids = torch.from_numpy(w.tables_np[b, :nblk].astype(np.int64)).to(w.key_cache.device)
            kvi = torch.tensor(kv, dtype=torch.int64, device=w.key_cache.device)
            smp["kc"] = bits_np(w.key_cache.index_select(0, ids).index_select(2, kvi))
            smp["vc"] = bits_np(w.value_cache.index_select(0, ids).index_select(2, kvi))
        eb = 1 if fp8 else 2
        smp["bytes"] = (L * len(kv) * cfg.head_dim * 2 * eb + (8 * L if fp8 else 0) + len(heads) * cfg.head_dim * 2
                        + nblk * 4 + 4)
        samples.append(smp)
    return samples


def cpu_baseline(pool, workers, cores, samples_by_config, seconds):
    """The oracle's rate on the host cores for every workload's sample (about ``seconds`` of work per
    workload on every worker).  tokens/s counts decoded sequence steps (a sample holding h of a
    sequence's H heads counts h / H of a step); GB/s is the algorithmic bytes the oracle's
    decodes cover, per second."""
    out = {}
    for name, samples in samples_by_config.items():
        order = sorted(samples, key=lambda s: -s["L"] * s["heads"])
        chunks = [order[i::workers] for i in range(workers)]
        chunks = [c for c in chunks if c]
        t0 = time.perf_counter()
        res = list(pool.map(_oracle_step_chunk, chunks, [seconds] * len(chunks)))
        wall = time.perf_counter() - t0
        tok_rate = sum(sum(s["heads"] / s["all_heads"] for s in c) * reps / el for c, (el, reps) in zip(chunks, res))
        byte_rate = sum(sum(s["bytes"] for s in c) * reps / el for c, (el, reps) in zip(chunks, res))
        per_worker = [sum(s["heads"] / s["all_heads"] for s in c) * reps / el for c, (el, reps) in zip(chunks, res)]
        rows = sum(s["heads"] for s in samples)
        out[name] = {"tokens_per_s": round(tok_rate, 3), "GBs": round(byte_rate / 1e9, 4),
                     "cores": len(chunks), "wall_s": round(wall, 1),
                     "per_core_tokens_per_s": round(sum(per_worker) / len(per_worker), 3),
                     "sample": f"{len(samples)} sequence(s), {rows} (sequence, head) row(s) of "
                               f"{samples[0]['all_heads']} head(s) each, split over {len(chunks)} worker process(es), "
                               f"each repeating its share's append + float64 decode for ~{seconds:g} s"}
    return out


# Heads per sequence in the CPU baseline's sample (0 or absent: every head).  The long-context
# workload's caches are 10.7 GB, so its sample is 2 seeded heads of each of its 8 sequences;
# the 256-sequence workload's 4.3 GB are sampled at 4 heads of each sequence.
CPU_SAMPLE_HEADS = {"longctx": 2, "llama7b_b256": 4}


def summarize(name, r):
    achieved = r["bytes"] / (r["decode_ms_mean"] * 1e-3) / 1e9
    cfg = r["w"].cfg
    return {
        "workload": name,
        "tokens_per_s": round(cfg.num_seqs * r.get("q_len", 1) / (r["ms_per_step"] * 1e-3), 1),
        "ms_per_step": round(r["ms_per_step"], 5),
        "step_gpu_us": round(r["step_gpu_ms"] * 1e3, 2),
        "decode_us_mean": round(r["decode_ms_mean"] * 1e3, 2),
        "decode_timing": r["decode_timing"],
        "decode_us_p10_p50_p90_per_call_events": [round(r[k] * 1e3, 2) for k in ("decode_ms_p10", "decode_ms_p50",
                                                                                   "decode_ms_p90")],
        "algorithmic_bytes": r["bytes"],
        "effective_GBs": round(achieved, 1),
        "frac_of_peak": round(achieved / HBM_PEAK_GBS, 4),
        "partition_size": r["partition_size"],
        "step": "pa_decode_append" if r.get("fused") else "pa_append_kv + decode call",
        **({"logical_bytes": logical_bytes(r["w"])} if cfg.beams > 1 else {}),
    }


def logical_bytes(w):
    """Bytes the decode requests when every sequence reads its own blocks (shared-prefix
    blocks counted once per beam); the % of peak is quoted on the unique bytes."""
    import numpy as np
    cfg = w.cfg
    eb = 1 if cfg.cache_dtype == "fp8_e4m3" else 2
    lens = w.lens_np.astype(np.int64)
    tokens = int(lens.sum())
    kv = tokens * cfg.num_kv_heads * cfg.head_dim * 2 * eb + (tokens * 8 if eb == 1 else 0)
    return kv + cfg.num_seqs * cfg.num_heads * cfg.head_dim * 2 + int(np.sum((lens + 15) // 16)) * 4 + cfg.num_seqs * 4


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama7b")
    ap.add_argument("--replicas", type=int, default=3, help="pool replicas rotated across steps")
    ap.add_argument("--also", default="gqa70b,fp8beams,longctx,llama7b_b256", help="comma-separated extra workloads reported alongside "
                    "(a workload with shared-prefix beams is also timed through pa_decode_shared_prefix)")
    ap.add_argument("--cpu-seconds", type=float, default=4.0,
                    help="oracle time per workload and worker for cpu_baseline (seconds)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graphs", action="store_true", help="replay captured HIP graphs of each replica's append "
                    "and decode instead of launching from Python (slower on ROCm 7 for this two-launch step)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (5 times), to scale rocprofv3 FETCH_SIZE/WRITE_SIZE")
    ap.add_argument("--no-copy", action="store_true", help="skip the pa_copy_blocks / pa_swap_blocks measurements")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the read-bandwidth ceiling probes")
    ap.add_argument("--multi", type=int, default=4,
                    help="new tokens per sequence of the extra pa_decode_multi line on the main workload; <2 = skip")
    ap.add_argument("--window", type=int, default=512,
                    help="sliding window (tokens) of the extra pa_decode_sliding line on the main workload; 0 = skip")
    ap.add_argument("--shared-prefix", action="store_true",
                    help="time the main workload (one with shared-prefix beams) through pa_decode_shared_prefix")
    ap.add_argument("--unfused", action="store_true",
                    help="time the step as pa_append_kv + pa_decode instead of pa_decode_append (one call); "
                         "the default run also reports the unfused step of the main workload")
    ap.add_argument("--no-unfused-line", action="store_true",
                    help="skip the unfused step of the main workload (counter runs of the fused step alone)")
    ap.add_argument("--partition-size", type=int, default=None,
                    help="override the workload's partition length (tokens; 0 = library's choice)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported (the library has no "
              "multi-GPU path; the paged decode would shard by sequence or KV head with no exchange)",
              file=sys.stderr)
        sys.exit(2)

    # The oracle's worker processes start before anything touches the GPU.
    oracle_pool = None if (args.no_cpu_baseline or args.calibrate_copy) else start_oracle_pool()

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device copy", "bytes_read_per_copy": 1 << 30,
                          "bytes_written_per_copy": 1 << 30, "copies": 5}), flush=True)
        return

    import paged_kv_cache_187_amd as pa
    import synth
    pa.load_library()

    if args.shared_prefix and synth.CONFIGS[args.workload].beams < 2:
        print(f"--shared-prefix needs a workload with shared-prefix beams, not {args.workload}", file=sys.stderr)
        sys.exit(2)
    def sample_of(name):
        """Heads kept per sequence in the CPU baseline's sample (0 = all), None without a baseline."""
        if oracle_pool is None:
            return None
        return CPU_SAMPLE_HEADS.get(name, 0)

    cpu_samples = {}
    fused = not (args.unfused or args.shared_prefix)
    main_r = time_workload(args.workload, args.steps, args.warmup, args.replicas, sample=sample_of(args.workload),
                           partition_size=args.partition_size, use_graphs=args.graphs,
                           shared_prefix=args.shared_prefix, fused=fused)
    s = summarize(args.workload, main_r)
    cfg = main_r["w"].cfg
    if oracle_pool is not None:
        cpu_samples[args.workload] = main_r["cpu_sample"]
    also = {}
    for name in [n for n in args.also.split(",") if n and n != args.workload]:
        r = time_workload(name, args.steps, args.warmup, args.replicas, sample=sample_of(name),
                          partition_size=args.partition_size, use_graphs=args.graphs, fused=fused)
        if oracle_pool is not None:
            cpu_samples[name] = r["cpu_sample"]
        also[name] = summarize(name, r)
        also[name]["traffic"] = measured_traffic(name)
        del r
        torch.cuda.empty_cache()
        if synth.CONFIGS[name].beams > 1:
            r = time_workload(name, args.steps, args.warmup, args.replicas, use_graphs=args.graphs,
                              shared_prefix=True)
            also[f"{name}_shared_prefix"] = summarize(name, r)
            also[f"{name}_shared_prefix"]["traffic"] = measured_traffic(f"{name}_shared_prefix")
            del r
            torch.cuda.empty_cache()

    if fused and not args.no_unfused_line:
        r = time_workload(args.workload, args.steps, args.warmup, args.replicas, partition_size=args.partition_size,
                          use_graphs=args.graphs)
        also[f"{args.workload}_unfused"] = summarize(args.workload, r)
        del r
        torch.cuda.empty_cache()
    if args.multi > 1:
        r = time_workload(args.workload, args.steps, args.warmup, args.replicas, partition_size=args.partition_size,
                          use_graphs=args.graphs, q_len=args.multi)
        also[f"{args.workload}_multi{args.multi}"] = summarize(args.workload, r)
        also[f"{args.workload}_multi{args.multi}"]["q_len"] = args.multi
        del r
        torch.cuda.empty_cache()
    if args.window > 0:
        r = time_workload(args.workload, args.steps, args.warmup, args.replicas, partition_size=args.partition_size,
                          use_graphs=args.graphs, window=args.window)
        also[f"{args.workload}_window{args.window}"] = summarize(args.workload, r)
        also[f"{args.workload}_window{args.window}"]["sliding_window"] = args.window
        del r
        torch.cuda.empty_cache()
    if not args.no_copy:
        also["copy_blocks"] = {"bandwidth": time_copy_blocks(args.steps, args.warmup, 1024),
                               "copy_on_write_64_pairs": time_copy_blocks(args.steps, args.warmup, 64)}
        also["swap_blocks"] = time_swap(min(args.steps, 50), min(args.warmup, 5))
        torch.cuda.empty_cache()

    ceiling = None if args.no_ceiling else read_ceiling()

    result = {
        "metric": METRIC,
        "value": s["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": s["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.cache_dtype,
        "data": "synthetic",
        "config": {
            "workload": WORKLOAD_TEXT.get(args.workload, args.workload),
            "num_seqs": cfg.num_seqs, "num_heads": cfg.num_heads, "num_kv_heads": cfg.num_kv_heads,
            "head_dim": cfg.head_dim, "block_size": 16, "kv_dtype": cfg.cache_dtype, "q_dtype": cfg.q_dtype,
            "accumulate": "f32", "partition_size": s["partition_size"], "pool_replicas": args.replicas,
            "hip_graphs": args.graphs,
            "step": ("one pa_decode_append call (append fused into the decode)" if fused
                     else "pa_append_kv + pa_decode" if not args.shared_prefix
                     else "pa_append_kv + pa_decode_shared_prefix"),
            "tokens_in_cache": int(main_r["w"].lens_np.sum()),
        },
        "roofline": {
            "kernel": ("pa_decode_append (decode_kernel with the append fused in + decode_merge_kernel)" if fused
                       else "pa_decode (decode_kernel + decode_merge_kernel)"),
            "bound": "hbm",
            "achieved": s["effective_GBs"],
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": s["frac_of_peak"],
            "traffic": measured_traffic(args.workload + ("_shared_prefix" if args.shared_prefix else "")),
            "bytes_per_launch": s["algorithmic_bytes"],
            "launch_us_mean": s["decode_us_mean"],
            "launch_timing": s["decode_timing"],
            "launch_us_p10_p50_p90_per_call_events": s["decode_us_p10_p50_p90_per_call_events"],
        },
        "also": also,
        # achievable read bandwidth on this GPU (probe kernels), labelled apart from the decode
        "ceiling": ceiling,
    }
    if oracle_pool is not None:
        pool, workers, host_cores, started = oracle_pool
        if "tiny" not in cpu_samples:
            cpu_samples["tiny"] = cpu_sample(synth.make_workload("tiny"))
        by_cfg = cpu_baseline(pool, workers, host_cores, cpu_samples, args.cpu_seconds)
        pool.shutdown()
        main_cpu = by_cfg[args.workload]
        result["cpu_baseline"] = {
            "value": main_cpu["tokens_per_s"], "unit": "tokens/s", "cores": main_cpu["cores"], "kind": "oracle",
            "sample": f"{args.workload}: {main_cpu['sample']}",
            "host_cores": host_cores, "worker_processes": started, "blas_threads_per_worker": 1,
            "by_config": by_cfg,
        }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
