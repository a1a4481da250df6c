"""The read-bandwidth probes behind bench.py's ceiling read exactly the bytes they claim.

Both probe kernels XOR every 32-bit word they load into one word per lane of a sink, so
the sink can be recomputed on the host from the same pool: a probe that skipped loads,
read the wrong rows or ran past its ranges would not match.
"""

import ctypes
import os

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


def _lib():
    from paged_kv_cache_187_amd.build import PROBE_PATH
    if not os.path.exists(PROBE_PATH):
        pytest.fail("libpaprobe.so is not built")
    lib = ctypes.CDLL(PROBE_PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.pa_probe_stream.argtypes = [vp, i64, vp, i32, vp]
    lib.pa_probe_gather.argtypes = [vp, vp, i32, i32, i32, i64, i32, vp, vp]
    lib.pa_probe_gather_teams.argtypes = [vp, vp, i32, i32, i32, i64, i32, vp, vp]
    return lib


def _say(msg):
    print(f"[case] {msg}", flush=True)


def _gather_expected(words, ids, hkv, row, num_blocks, waves):
    """Per (wave, lane) XOR of the words the gather probe loads: for each (head, block)
    pair of the wave's range, the 16 rows of that head, each lane owning 16 bytes of a row."""
    tok = hkv * row // 4                       # in words
    blk = 16 * tok
    lpr = row // 16                            # lanes per row
    rpl = 64 // lpr                            # rows per load
    n_ids = len(ids)
    T = hkv * n_ids
    C = -(-T // waves)
    lane = np.arange(64)
    base = (lane // lpr) * tok + (lane % lpr) * 4
    out = np.zeros((waves, 64), dtype=np.uint32)
    for w in range(waves):
        lo, hi = min(w * C, T), min(w * C + C, T)
        acc = np.zeros(64, dtype=np.uint32)
        for q in range(lo, hi):
            head, i = divmod(q, n_ids)
            bid = int(ids[i])
            if bid < 0 or bid >= num_blocks:
                bid = 0
            for ld in range(16 // rpl):
                off = bid * blk + ld * rpl * tok + head * row // 4 + base
                for k in range(4):
                    acc ^= words[off + k]
        out[w] = acc
    return out


def _gather_teams_expected(words, ids, hkv, row, num_blocks, waves):
    """The same XOR for the team order: wave w reads head w % hkv of id range w / hkv, the
    ranges [r n / teams, (r + 1) n / teams) of the n ids."""
    tok = hkv * row // 4
    blk = 16 * tok
    lpr = row // 16
    rpl = 64 // lpr
    n_ids = len(ids)
    teams = waves // hkv
    lane = np.arange(64)
    base = (lane // lpr) * tok + (lane % lpr) * 4
    out = np.zeros((waves, 64), dtype=np.uint32)
    for w in range(waves):
        head, r = w % hkv, w // hkv
        acc = np.zeros(64, dtype=np.uint32)
        for i in range(r * n_ids // teams, (r + 1) * n_ids // teams):
            bid = int(ids[i])
            if bid < 0 or bid >= num_blocks:
                bid = 0
            for ld in range(16 // rpl):
                off = bid * blk + ld * rpl * tok + head * row // 4 + base
                for k in range(4):
                    acc ^= words[off + k]
        out[w] = acc
    return out


@pytest.mark.parametrize("row,hkv,n_ids,waves", [
    (128, 3, 37, 9),        # waves not a multiple of the 4 per workgroup
    (256, 2, 29, 200),      # more teams than blocks: empty ranges
    (128, 8, 64, 16),
    (256, 8, 23, 64),
])
def test_gather_teams_probe_reads_every_row_it_claims(row, hkv, n_ids, waves):
    _say(f"gather probe (teams) row={row} hkv={hkv} ids={n_ids} waves={waves}")
    lib = _lib()
    num_blocks = 50
    rng = np.random.default_rng(row + hkv + n_ids + 1)
    words = rng.integers(0, 1 << 32, size=num_blocks * 16 * hkv * row // 4, dtype=np.uint64).astype(np.uint32)
    ids = rng.integers(0, num_blocks, size=n_ids).astype(np.int32)
    ids[3] = -1                                # outside the pool: the probe reads block 0
    ids[5] = num_blocks + 4
    pool = torch.from_numpy(words.view(np.int32).copy()).cuda()
    dids = torch.from_numpy(ids).cuda()
    sink = torch.zeros(waves * 64, dtype=torch.int32, device="cuda")
    assert lib.pa_probe_gather_teams(pool.data_ptr(), dids.data_ptr(), n_ids, hkv, row, num_blocks, waves,
                                     sink.data_ptr(), None) == 0
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32).reshape(waves, 64)
    np.testing.assert_array_equal(got, _gather_teams_expected(words, ids, hkv, row, num_blocks, waves))


@pytest.mark.parametrize("row,hkv,n_ids,waves", [
    (128, 3, 37, 7),        # waves not a multiple of the 4 per workgroup
    (256, 2, 29, 200),      # more waves than (head, block) pairs: empty ranges
    (128, 8, 64, 16),
    (256, 5, 23, 13),
])
def test_gather_probe_reads_every_row_it_claims(row, hkv, n_ids, waves):
    _say(f"gather probe row={row} hkv={hkv} ids={n_ids} waves={waves}")
    lib = _lib()
    num_blocks = 50
    rng = np.random.default_rng(row + hkv + n_ids)
    words = rng.integers(0, 1 << 32, size=num_blocks * 16 * hkv * row // 4, dtype=np.uint64).astype(np.uint32)
    ids = rng.integers(0, num_blocks, size=n_ids).astype(np.int32)
    ids[3] = -1                                # outside the pool: the probe reads block 0
    ids[5] = num_blocks + 4
    pool = torch.from_numpy(words.view(np.int32).copy()).cuda()
    dids = torch.from_numpy(ids).cuda()
    sink = torch.zeros(waves * 64, dtype=torch.int32, device="cuda")
    assert lib.pa_probe_gather(pool.data_ptr(), dids.data_ptr(), n_ids, hkv, row, num_blocks, waves,
                               sink.data_ptr(), None) == 0
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32).reshape(waves, 64)
    np.testing.assert_array_equal(got, _gather_expected(words, ids, hkv, row, num_blocks, waves))


def test_stream_probe_reads_the_whole_buffer():
    _say("stream probe: 1 MiB + 48 bytes over 3 workgroups")
    lib = _lib()
    nbytes = (1 << 20) + 48
    blocks = 3
    rng = np.random.default_rng(5)
    words = rng.integers(0, 1 << 32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(words.view(np.int32).copy()).cuda()
    sink = torch.zeros(blocks * 256, dtype=torch.int32, device="cuda")
    assert lib.pa_probe_stream(buf.data_ptr(), nbytes, sink.data_ptr(), blocks, None) == 0
    torch.cuda.synchronize()
    vec = words.reshape(-1, 4)
    per = np.bitwise_xor.reduce(vec, axis=1)                  # XOR of each 16-byte vector
    threads = blocks * 256
    pad = (-len(per)) % threads
    expected = np.bitwise_xor.reduce(np.concatenate([per, np.zeros(pad, np.uint32)]).reshape(-1, threads), axis=0)
    np.testing.assert_array_equal(sink.cpu().numpy().view(np.uint32), expected)
