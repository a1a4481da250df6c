"""Oracle of the slot-mapped KV append (reshape_and_cache) and its FP8 variant.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources:

* "大模型推理引擎优化：KV Cache 与连续批处理" (devpress.csdn.net), §2.1: each decode step
  adds the new token's K and V to the cache that later steps read; §2.2 and the
  block manager of §三: blocks hold 16 tokens, a sequence that outgrows its last
  block gets a fresh one on demand, so the new token of a sequence whose length
  becomes n lands at offset (n-1) mod 16 of its block number (n-1) div 16.
* "LLM推理引擎深度实战：从PagedAttention到分布式推理部署", §2.2 (16-token pages, allocated
  only for tokens that exist) and §5.3 (FP8 KV cache at per-token granularity).

Slot encoding (a reading; the pages return only a block from the append): a
slot is ``physical_block * 16 + offset``; a slot outside [0, 16 * num_blocks)
(negative for padding tokens, or past the pool) means "write nothing" for
that token.

Pools are bit-pattern arrays shaped [num_blocks, 16, num_kv_heads, head_dim]:
uint16 for float16 / bfloat16 caches and uint8 codes for the FP8 cache, with
per-token float32 scales shaped [num_blocks, 16].  Every function returns new
arrays and leaves its arguments untouched.
"""

import numpy as np

from .codecs import decode_bits, encode_e4m3, E4M3_MAX

BLOCK_SIZE = 16


def append_kv(key_cache, value_cache, key, value, slot_mapping):
    """Copy token t's K/V rows ([Hkv, D] bit patterns) into slot slot_mapping[t].

    key/value: [T, Hkv, D] arrays of the cache's bit-pattern dtype.  Tokens are
    written in order t = 0..T-1 with plain numpy element assignment.
    """
    kc = np.array(key_cache, copy=True)
    vc = np.array(value_cache, copy=True)
    num_slots = kc.shape[0] * BLOCK_SIZE
    for t, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if slot < 0 or slot >= num_slots:
            continue
        blk, off = divmod(int(slot), BLOCK_SIZE)
        kc[blk, off] = key[t]
        vc[blk, off] = value[t]
    return kc, vc


def quantize_tokens_e4m3(x):
    """Per-token FP8 E4M3 quantisation of float32 rows.

    x: float32 [T, N] (one token's Hkv*D elements per row; here the exact
    float32 values of bfloat16 / float16 inputs).  For each row:

        amax  = max |x|                     (float32, exact)
        scale = amax / 448                  (IEEE float32 division, RNE);
                scale = 1 when amax == 0
        code  = E4M3(float32(x / scale))    (float32 division, then RNE and
                                             saturation to +-448)

    The scale is per token and shared by all heads and channels of that token
    (reading of "per-token granularity", §5.3 of the ybb.press page).
    Returns (codes uint8 [T, N], scales float32 [T]).
    """
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=1).astype(np.float32) if x.shape[1] else np.zeros(x.shape[0], np.float32)
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    scale = np.where(amax == 0, np.float32(1.0), scale).astype(np.float32)
    y = (x / scale[:, None]).astype(np.float32)
    return encode_e4m3(y), scale


def append_kv_e4m3(key_cache, value_cache, k_scale, v_scale, key, value, src_dtype, slot_mapping):
    """Quantising append: K and V of each token are quantised separately.

    key/value: [T, Hkv, D] uint16 bit patterns of ``src_dtype`` ("f16" or
    "bf16").  Caches are uint8 [nb, 16, Hkv, D]; scales float32 [nb, 16].
    """
    T = key.shape[0]
    kf = decode_bits(key, src_dtype).astype(np.float32).reshape(T, -1)  # exact
    vf = decode_bits(value, src_dtype).astype(np.float32).reshape(T, -1)
    kq, ks = quantize_tokens_e4m3(kf)
    vq, vs = quantize_tokens_e4m3(vf)
    kc = np.array(key_cache, copy=True)
    vc = np.array(value_cache, copy=True)
    ksc = np.array(k_scale, copy=True)
    vsc = np.array(v_scale, copy=True)
    row_shape = key_cache.shape[2:]
    num_slots = key_cache.shape[0] * BLOCK_SIZE
    for t, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if slot < 0 or slot >= num_slots:
            continue
        blk, off = divmod(int(slot), BLOCK_SIZE)
        kc[blk, off] = kq[t].reshape(row_shape)
        vc[blk, off] = vq[t].reshape(row_shape)
        ksc[blk, off] = ks[t]
        vsc[blk, off] = vs[t]
    return kc, vc, ksc, vsc
