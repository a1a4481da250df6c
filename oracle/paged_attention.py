"""Oracle of paged decode attention, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed ("LLM推理引擎深度实战：从PagedAttention到分布式推理部署", §2.2-§2.3; "大模型推理
引擎优化：KV Cache 与连续批处理", §2.1-§2.2): in a decode step each sequence's single
new query token attends over the K/V of all of its tokens.  Those K/V rows sit
in 16-token physical blocks, and the page table of the sequence maps its
logical block j to a physical block.  Paging is transparent: the result is
plain softmax attention over the tokens in logical order.  Per sequence b and
query head h:

    g        = Hq / Hkv ;  kv head of h = h // g        (reading: consecutive
                                                          query heads share a
                                                          KV head)
    K[t], V[t] = rows (t mod 16) of physical block block_tables[b][t // 16],
                 kv head h // g, for t = 0 .. L_b - 1
                 (FP8 cache: code value times that token's scale)
    s[t]     = scale * <q[b, h], K[t]>
    w        = exp(s - max s) / sum(exp(s - max s))
    out[b,h] = sum_t w[t] V[t]            (zeros when L_b == 0)

The gather into contiguous K/V is done first, then the attention, as the
plain definition reads; numpy matrix products are the only library steps.

Several new tokens per sequence ("LLM推理引擎深度实战：…", §6.1: the large model
checks γ speculative tokens in one forward pass; "大模型推理引擎优化：…", §4.1: chunked
prefill runs a long input a chunk at a time): with Q new tokens appended, the
sequence holds L tokens and new token i (0 <= i < Q) sits at position
L - Q + i.  Reading (causal attention, as the forward pass over those tokens
computes): its query attends to tokens 0 .. L - Q + i, so new tokens see the
cache and the new tokens before them, never those after.

Sliding window ("LLM推理引擎深度实战：…", §9.2 names sliding-window attention, as in
Mistral, among the long-context methods without defining it; the reading taken
is the usual one): with a window of W > 0 tokens the query of a sequence of
length L attends only to its last W tokens, t = max(0, L - W) .. L - 1 (itself
included).  W = 0 means no window.
"""

import numpy as np

from .codecs import decode_bits

BLOCK_SIZE = 16


def attention_weights(q, K, scale):
    """Softmax weights of one query over L keys: float64 [L]."""
    s = scale * (K @ q)
    e = np.exp(s - np.max(s))
    return e / np.sum(e)


def attend(q, K, V, scale):
    """Single-query attention over contiguous keys/values (float64).

    q [D], K [L, D], V [L, D] -> [D]; zeros for L == 0.
    """
    if K.shape[0] == 0:
        return np.zeros(V.shape[1], dtype=np.float64)
    return attention_weights(q, K, scale) @ V


def gather_kv(cache_bits, block_table, length, dtype, scales=None):
    """Gather the first ``length`` tokens of one sequence into contiguous float64 rows.

    cache_bits: [num_blocks, 16, Hkv, D] bit patterns of ``dtype``; block_table:
    the sequence's logical->physical block ids; scales: optional float32
    [num_blocks, 16] per-token multipliers (FP8 cache).  Token t is row
    t mod 16 of physical block block_table[t div 16].  Returns [L, Hkv, D].
    """
    rows = []
    mult = []
    for t in range(length):
        phys = int(block_table[t // BLOCK_SIZE])
        off = t % BLOCK_SIZE
        rows.append(cache_bits[phys, off])
        if scales is not None:
            mult.append(float(scales[phys, off]))
    if not rows:
        return np.zeros((0,) + tuple(cache_bits.shape[2:]), dtype=np.float64)
    out = decode_bits(np.stack(rows), dtype)
    if scales is not None:
        out = out * np.array(mult, dtype=np.float64)[:, None, None]
    return out


def window_start(length, window):
    """First token a query attends to: max(0, L - W) with a window of W > 0 tokens, else 0."""
    return max(0, length - window) if window > 0 else 0


def paged_decode(query, key_cache, value_cache, block_tables, context_lens, scale,
                 q_dtype, cache_dtype, k_scale=None, v_scale=None, window=0):
    """Paged decode attention for a whole batch.

    query: [B, Hq, D] bit patterns (uint16) of ``q_dtype``; caches:
    [num_blocks, 16, Hkv, D] bit patterns of ``cache_dtype`` ("f16", "bf16",
    or "fp8_e4m3" with float32 k_scale / v_scale [num_blocks, 16]);
    block_tables: int [B, max_blocks]; context_lens: int [B]; window: sliding
    window in tokens (0 = none).  Returns float64 [B, Hq, D].
    """
    q = decode_bits(query, q_dtype)
    B, Hq, D = q.shape
    Hkv = key_cache.shape[2]
    g = Hq // Hkv
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        L = int(context_lens[b])
        lo = window_start(L, window)
        K = gather_kv(key_cache, block_tables[b], L, cache_dtype, k_scale)[lo:]
        V = gather_kv(value_cache, block_tables[b], L, cache_dtype, v_scale)[lo:]
        for h in range(Hq):
            out[b, h] = attend(q[b, h], K[:, h // g, :], V[:, h // g, :], scale)
    return out


def paged_decode_multi(query, key_cache, value_cache, block_tables, context_lens, scale,
                       q_dtype, cache_dtype, k_scale=None, v_scale=None):
    """Paged attention of Q new tokens per sequence, causal within the new chunk.

    query: [B, Q, Hq, D] bit patterns of ``q_dtype``; context_lens [B] count the Q new tokens.
    Query i of sequence b attends to tokens 0 .. L_b - Q + i (zeros if that range is empty).
    Returns float64 [B, Q, Hq, D].
    """
    q = decode_bits(query, q_dtype)
    B, Q, Hq, D = q.shape
    Hkv = key_cache.shape[2]
    g = Hq // Hkv
    out = np.zeros((B, Q, Hq, D), dtype=np.float64)
    for b in range(B):
        L = int(context_lens[b])
        K = gather_kv(key_cache, block_tables[b], L, cache_dtype, k_scale)
        V = gather_kv(value_cache, block_tables[b], L, cache_dtype, v_scale)
        for i in range(Q):
            last = L - Q + i                  # position of new token i; it sees tokens 0..last
            n = max(0, last + 1)
            for h in range(Hq):
                out[b, i, h] = attend(q[b, i, h], K[:n, h // g, :], V[:n, h // g, :], scale)
    return out


def paged_decode_one(q_vec, key_cache, value_cache, block_table, length, kv_head, scale,
                     cache_dtype, k_scale=None, v_scale=None, window=0):
    """One (sequence, head) of ``paged_decode``, for sampled checks of large runs.

    q_vec: float64 [D] (already decoded); caches are bit-pattern arrays that
    need only hold the blocks ``block_table`` names.
    """
    lo = window_start(length, window)
    K = gather_kv(key_cache, block_table, length, cache_dtype, k_scale)[lo:]
    V = gather_kv(value_cache, block_table, length, cache_dtype, v_scale)[lo:]
    return attend(np.asarray(q_vec, dtype=np.float64), K[:, kv_head, :], V[:, kv_head, :], scale)


def partial_attend(q, K, V, scale):
    """Unnormalised attention over one partition of the keys.

    Returns (m, l, acc): m = max score, l = sum exp(s - m), acc = sum exp(s - m) V.
    An empty partition returns (-inf, 0, zeros).
    """
    if K.shape[0] == 0:
        return -np.inf, 0.0, np.zeros(V.shape[1], dtype=np.float64)
    s = scale * (K @ q)
    m = np.max(s)
    e = np.exp(s - m)
    return m, np.sum(e), e @ V


def merge_partials(parts):
    """Log-sum-exp merge of partition results [(m, l, acc), ...] in list order.

    out = sum_p exp(m_p - M) acc_p / sum_p exp(m_p - M) l_p with M = max_p m_p;
    zeros when every partition is empty.
    """
    ms = np.array([p[0] for p in parts], dtype=np.float64)
    if len(parts) == 0 or not np.isfinite(ms).any():
        D = parts[0][2].shape[0] if parts else 0
        return np.zeros(D, dtype=np.float64)
    M = np.max(ms)
    num = 0.0
    den = 0.0
    for m, l, acc in parts:
        if not np.isfinite(m):
            continue
        w = np.exp(m - M)
        num = num + w * acc
        den = den + w * l
    return num / den
