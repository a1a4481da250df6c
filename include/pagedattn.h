/*
 * pagedattn.h - C ABI of the gfx950 (MI355X) paged decode attention library.
 *
 * The operations, all from the pages' description of PagedAttention:
 *
 *  - pa_append_kv: write each new token's K and V rows into the slot of the
 *    KV cache that the block manager gave it ("大模型推理引擎优化：KV Cache 与连续批处理",
 *    §2.1 and §2.2: every decode step adds the new token's K/V, in 16-token
 *    blocks handed out on demand), optionally quantising them to FP8 E4M3
 *    with one float32 scale per token ("LLM推理引擎深度实战：从PagedAttention到分布式推理部署",
 *    §5.3: FP8 KV cache, per-token granularity).
 *
 *  - pa_decode: one query token per sequence attends over that sequence's
 *    cached K/V, which sit in fixed 16-token physical blocks reached through
 *    the sequence's page table; the kernel turns logical token indices into
 *    physical addresses, so the result is plain softmax attention over the
 *    tokens in logical order ("LLM推理引擎深度实战：…", §2.2 and §2.3);
 *    pa_decode_sliding restricts it to a sliding window of recent tokens;
 *    pa_decode_multi takes several new tokens per sequence (causal).
 *
 *  - pa_decode_append: both in one call (the append fused into the decode).
 *
 *  - pa_copy_blocks: copy whole physical blocks, the copy-on-write step the
 *    block manager takes before a sequence writes into a block that other
 *    sequences share ("大模型推理引擎优化：…", §4.2; "LLM推理引擎深度实战：…", §2.2).
 *
 *  - pa_swap_blocks: the same copy between two pools, one of which may be
 *    pinned host memory: a preempted request's blocks go out to CPU memory and
 *    come back when it resumes ("LLM推理引擎深度实战：…", §3.2).
 *
 * Layouts (all row-major, contiguous, little-endian):
 *   query        [num_seqs, num_heads, head_dim]                 q_dtype
 *   out          [num_seqs, num_heads, head_dim]                 q_dtype
 *   key_cache    [num_blocks, 16, num_kv_heads, head_dim]        cache_dtype
 *   value_cache  [num_blocks, 16, num_kv_heads, head_dim]        cache_dtype
 *   k_scale      [num_blocks, 16] float32   (FP8 cache only; one scale per token slot)
 *   v_scale      [num_blocks, 16] float32   (FP8 cache only)
 *   block_tables [num_seqs, max_blocks_per_seq] int32: physical block of
 *                logical block j of sequence b
 *   context_lens [num_seqs] int32: tokens of sequence b, including the one
 *                appended in this step
 *   slot_mapping [num_tokens] int64: physical_block * 16 + offset; < 0 = skip
 *
 * Query head h reads KV head h / (num_heads / num_kv_heads) (consecutive
 * query heads share a KV head).  Block size is fixed at 16 tokens.
 *
 * Ownership and ordering: every pointer argument is a caller-owned device
 * buffer (except where noted); the library allocates nothing, keeps nothing
 * after a call returns and has no mutable global state, so it may be called
 * from several threads.  The one exception is pa_decode_noalloc, whose
 * partial results live in a fixed device array per GPU (see there).  Work is enqueued asynchronously on `stream` (a
 * hipStream_t; NULL = the null stream); an append followed by a decode on
 * the same stream is ordered.  Host-side argument checks run before anything
 * is enqueued and never read device memory, so no call synchronises.
 *
 * Errors: functions return a pa_status.  PA_ERR_* codes other than
 * PA_ERR_HIP come from host-side checks and leave every buffer untouched.
 * PA_ERR_HIP reports a launch failure (hipGetLastError after the launch).
 * Device contents are the caller's contract: slots and table entries that
 * fall outside [0, num_blocks) are ignored by the kernels (that token or block
 * is skipped, never read or written), and context_lens are clamped to
 * [0, min(max_context_len, 16 * max_blocks_per_seq)].
 */
#ifndef PAGEDATTN_H
#define PAGEDATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_BLOCK_SIZE 16

typedef enum pa_status {
    PA_OK = 0,
    PA_ERR_NULL = 1,        /* a required pointer is NULL                        */
    PA_ERR_SHAPE = 2,       /* a size is out of range or inconsistent            */
    PA_ERR_DTYPE = 3,       /* unsupported dtype or dtype combination            */
    PA_ERR_UNSUPPORTED = 4, /* head_dim or head grouping the kernels do not cover */
    PA_ERR_WORKSPACE = 5,   /* workspace missing or smaller than required        */
    PA_ERR_HIP = 6,         /* the HIP runtime reported an error                 */
    PA_ERR_ALIGN = 7,       /* a buffer is not 16-byte aligned                   */
    PA_ERR_ADDRESS = 8,     /* a buffer is not addressable by the GPU            */
    PA_ERR_SCRATCH = 9      /* pa_decode_noalloc: the call needs more workspace
                               than PA_NOALLOC_SCRATCH_BYTES                      */
} pa_status;

/* Size of the fixed device scratch behind pa_decode_noalloc (per GPU). */
#define PA_NOALLOC_SCRATCH_BYTES (64u << 20)

typedef enum pa_dtype {
    PA_F16 = 0,       /* IEEE binary16                                  */
    PA_BF16 = 1,      /* bfloat16                                       */
    PA_FP8_E4M3 = 2,  /* OCP FP8 E4M3 (fn): bias 7, max 448, no Inf      */
    PA_F32 = 3        /* listed for completeness; no operation takes it */
} pa_dtype;

/*
 * pa_append_kv - slot-mapped KV append (reshape_and_cache).
 *
 * For each token t < num_tokens with s = slot_mapping[t] in
 * [0, 16 * num_blocks): block = s / 16, offset = s % 16, and
 *   key_cache[block, offset, :, :]   <- key[t, :, :]
 *   value_cache[block, offset, :, :] <- value[t, :, :]
 * Tokens with s outside that range are skipped.
 *
 * key, value: [num_tokens, num_kv_heads, head_dim] of src_dtype.
 * cache_dtype == src_dtype (PA_F16 or PA_BF16): a bit-exact copy; k_scale and
 *   v_scale are ignored (may be NULL).
 * cache_dtype == PA_FP8_E4M3 (src PA_F16 or PA_BF16): K and V of each token
 *   are quantised separately over all num_kv_heads*head_dim elements:
 *   amax = max|x| (float32), scale = amax / 448 (IEEE float32 division;
 *   1.0 when amax == 0), code = E4M3(x / scale) with the division in float32,
 *   round-to-nearest-even and saturation to +-448; the codes go to the cache
 *   and the scales to k_scale[block, offset] / v_scale[block, offset].
 *
 * Two tokens with the same slot in one call race (undefined which wins).
 * head_dim must be 64 or 128.  All buffers 16-byte aligned (scales 4-byte).
 */
pa_status pa_append_kv(const void *key, const void *value,
                       void *key_cache, void *value_cache,
                       float *k_scale, float *v_scale,
                       const int64_t *slot_mapping,
                       int64_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                       int64_t num_blocks,
                       int32_t src_dtype, int32_t cache_dtype,
                       void *stream);

/*
 * pa_copy_blocks - for every pair i < num_pairs with (src, dst) =
 * (block_mapping[2 i], block_mapping[2 i + 1]): copy physical block src of
 * key_cache to block dst, likewise for value_cache, and for an FP8 cache the
 * block's 16 scales of k_scale and of v_scale, bit for bit.
 *
 * block_mapping: [num_pairs, 2] int64, device.  Pairs with src or dst outside
 * [0, num_blocks), or src == dst, are skipped.  The destinations of one call
 * must be distinct and must not be the source of another pair in the same
 * call (otherwise which bytes a block ends up with is undefined).  cache_dtype
 * F16, BF16 or FP8_E4M3 (k_scale / v_scale required for FP8, ignored
 * otherwise).  head_dim 64 or 128.  Caches 16-byte aligned, block_mapping
 * 8-byte aligned, scales 4-byte aligned.
 */
pa_status pa_copy_blocks(void *key_cache, void *value_cache,
                         float *k_scale, float *v_scale,
                         const int64_t *block_mapping, int64_t num_pairs,
                         int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks,
                         int32_t cache_dtype, void *stream);

/*
 * pa_swap_blocks - for every pair i < num_pairs with (src, dst) =
 * (block_mapping[2 i], block_mapping[2 i + 1]): copy block src of the source
 * pools (src_key, src_value and, for an FP8 cache, src_k_scale / src_v_scale)
 * to block dst of the destination pools, bit for bit.
 *
 * Either side may be pinned host memory the GPU can address (hipHostMalloc'd,
 * e.g. a torch tensor created with pin_memory=True); the copy then crosses
 * PCIe.  Every buffer is checked on the host with hipPointerGetAttributes
 * (which does not synchronise): one that the GPU cannot reach at the same
 * address returns PA_ERR_ADDRESS and nothing is launched.  block_mapping lives in device memory (or pinned host memory).  Pairs
 * with src outside [0, src_num_blocks) or dst outside [0, dst_num_blocks) are
 * skipped; the destinations of one call must be distinct.  Both sides have
 * the layout of key_cache / value_cache ([*_num_blocks, 16, num_kv_heads,
 * head_dim], cache_dtype) and of the scales; alignment as pa_copy_blocks.
 */
pa_status pa_swap_blocks(const void *src_key, const void *src_value,
                         const float *src_k_scale, const float *src_v_scale,
                         int64_t src_num_blocks,
                         void *dst_key, void *dst_value,
                         float *dst_k_scale, float *dst_v_scale,
                         int64_t dst_num_blocks,
                         const int64_t *block_mapping, int64_t num_pairs,
                         int32_t num_kv_heads, int32_t head_dim,
                         int32_t cache_dtype, void *stream);

/*
 * pa_decode_partition_size - how pa_decode splits the work for these
 * arguments.  partition_size > 0 (a multiple of 16, at most 2^20): fixed
 * partitions of that many tokens, one wave per (sequence, head group,
 * partition); the function returns partition_size.  partition_size == 0:
 * the balanced split, which cuts the (sequence, head group, 16-token block)
 * space into equal ranges, one per wave, whatever the length mix; the
 * function returns 0.  Returns -1 when the arguments are invalid.
 */
int32_t pa_decode_partition_size(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_context_len,
                                 int32_t partition_size);

/*
 * pa_decode_workspace_bytes - device workspace pa_decode needs for these
 * arguments, whatever the cache dtype ((size_t)-1 for invalid arguments; 0
 * when nothing is split, i.e. fixed partitions with max_context_len <=
 * partition_size).  The balanced split runs 1024 waves, or 2048 for an FP8 cache
 * (shared-prefix groups: 1024 always); the size returned is the larger one's.  The
 * workspace holds float32 partial results: per (slot, head of the group) a
 * V sum of head_dim floats, followed by all (max, sum of exponentials)
 * pairs.  Its contents need no initialisation and are scratch after the call;
 * calls that share a workspace must not run concurrently.
 */
size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_context_len,
                                 int32_t partition_size);

/*
 * pa_decode - paged decode attention, one query token per sequence.
 *
 * For each sequence b with L = context_lens[b] (clamped as above) and each
 * query head h, with g = num_heads / num_kv_heads and kv = h / g:
 *   K[t], V[t] = row (t % 16) of physical block block_tables[b, t / 16], KV
 *                head kv, for t < L (FP8 cache: code value * k_scale / v_scale
 *                of that slot)
 *   out[b, h, :] = sum_t softmax_t(scale * <query[b, h, :], K[t]>) V[t, :]
 * computed with float32 accumulation and rounded to q_dtype (round to nearest
 * even).  L == 0 gives a zero row.  Only slots t < L are read: whatever the
 * other slots and the table entries past ceil(L/16) hold never reaches out.
 *
 * Work is split over waves as pa_decode_partition_size describes; a
 * sequence covered by more than one wave gets partial results (running
 * max, sum of exponentials, weighted V sum) in `workspace` that a second
 * kernel merges in ascending token order, so for fixed inputs and fixed
 * (num_seqs, num_heads, num_kv_heads, head_dim, max_context_len,
 * partition_size) the output is bitwise deterministic.
 *
 * Alignment: query, out, caches and workspace 16 bytes; block_tables,
 * context_lens and k_scale / v_scale (FP8 cache) 4 bytes.
 *
 * Supported (q_dtype, cache_dtype): (F16, F16), (BF16, BF16), (F16, FP8_E4M3),
 * (BF16, FP8_E4M3).  head_dim 64 or 128.  num_heads a multiple of
 * num_kv_heads.  k_scale / v_scale required for FP8, ignored otherwise.
 * max_context_len: a host-side upper bound of context_lens, used to size the
 * partition grid.  workspace: device buffer of at least
 * pa_decode_workspace_bytes(...) bytes (may be NULL when that is 0); out must
 * not alias any input.
 */
pa_status pa_decode(void *out, const void *query,
                    const void *key_cache, const void *value_cache,
                    const float *k_scale, const float *v_scale,
                    const int32_t *block_tables, const int32_t *context_lens,
                    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                    int32_t head_dim, int64_t num_blocks,
                    int32_t max_blocks_per_seq, int32_t max_context_len,
                    float scale, int32_t partition_size,
                    int32_t q_dtype, int32_t cache_dtype,
                    void *workspace, size_t workspace_bytes,
                    void *stream);

/*
 * pa_decode_append - one whole decode step in one call: the slot-mapped append of each
 * sequence's new token ("大模型推理引擎优化：KV Cache 与连续批处理", §2.1-§2.2: each step adds
 * the new token's K/V to the cache the step attends over), then pa_decode over the cache
 * that now holds it.
 *
 * Sequence b with L = context_lens[b] (clamped as for pa_decode) > 0 has its new token at
 * position L - 1: row (L - 1) % 16 of physical block block_tables[b, (L - 1) / 16].
 * key_new / value_new: [num_seqs, num_kv_heads, head_dim] in q_dtype.  For a 16-bit cache
 * (cache_dtype == q_dtype) the rows are copied bit for bit; for an FP8 cache they are
 * quantised exactly as pa_append_kv quantises them (per-token scale amax / 448 over all
 * num_kv_heads * head_dim values, written to k_scale / v_scale).  Afterwards the caches (and
 * scales) are bit for bit what pa_append_kv with slot_mapping[b] = block * 16 + offset of
 * that position (negative for L == 0) leaves, and `out` is bit for bit what pa_decode then
 * returns.  Sequences with L == 0 append nothing; a table entry outside [0, num_blocks) is
 * not written.  The kernels take the new token's K/V from key_new / value_new, not from its
 * slot, so the slot's old contents never reach `out`; the block holding a new token must not
 * be read by another sequence in the same call (a block is private before anyone writes into
 * it: copy-on-write, pa_copy_blocks).  Every other argument, the workspace
 * (pa_decode_workspace_bytes), determinism and errors are those of pa_decode; key_new and
 * value_new must be 16-byte aligned (PA_ERR_ALIGN) and non-null (PA_ERR_NULL).
 */
pa_status pa_decode_append(void *out, const void *query,
                           const void *key_new, const void *value_new,
                           void *key_cache, void *value_cache,
                           float *k_scale, float *v_scale,
                           const int32_t *block_tables, const int32_t *context_lens,
                           int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                           int32_t head_dim, int64_t num_blocks,
                           int32_t max_blocks_per_seq, int32_t max_context_len,
                           float scale, int32_t partition_size,
                           int32_t q_dtype, int32_t cache_dtype,
                           void *workspace, size_t workspace_bytes,
                           void *stream);

/*
 * pa_decode_noalloc - pa_decode for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 *
 * Arguments, result, determinism and errors are those of pa_decode, without the
 * workspace: the partial results live in a fixed device array of
 * PA_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on until the
 * process ends (resolved once per device, on the first call with that device current;
 * `stream` must belong to the current device).  The call allocates nothing: no hipMalloc,
 * no hipFree, no allocating library routine.  A call whose pa_decode_workspace_bytes(...)
 * exceeds PA_NOALLOC_SCRATCH_BYTES returns PA_ERR_SCRATCH before anything is enqueued.
 * All calls on one GPU share that GPU's array (it keeps the last call's partials; nothing
 * in it needs to start at zero): calls that can overlap on one GPU (other streams, other
 * threads) race and must be serialised by the caller; pa_decode with its own workspace
 * has no such limit.  PA_ERR_HIP also reports a failure to resolve the array's address.
 */
pa_status pa_decode_noalloc(void *out, const void *query,
                            const void *key_cache, const void *value_cache,
                            const float *k_scale, const float *v_scale,
                            const int32_t *block_tables, const int32_t *context_lens,
                            int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                            int32_t head_dim, int64_t num_blocks,
                            int32_t max_blocks_per_seq, int32_t max_context_len,
                            float scale, int32_t partition_size,
                            int32_t q_dtype, int32_t cache_dtype,
                            void *stream);

/*
 * pa_decode_sliding - pa_decode with a sliding window: the query of a
 * sequence of length L attends only to its last sliding_window tokens,
 * t = max(0, L - sliding_window) .. L - 1 ("LLM推理引擎深度实战：…", §9.2 names
 * sliding-window attention among the long-context methods).  Only the blocks
 * holding those tokens are read; tokens before the window are excluded by
 * selection, so whatever their slots hold never reaches out.
 * sliding_window == 0 is pa_decode; negative values return PA_ERR_SHAPE.
 * Every other argument, the workspace (same pa_decode_workspace_bytes) and
 * the determinism guarantee are those of pa_decode.
 */
pa_status pa_decode_sliding(void *out, const void *query,
                            const void *key_cache, const void *value_cache,
                            const float *k_scale, const float *v_scale,
                            const int32_t *block_tables, const int32_t *context_lens,
                            int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                            int32_t head_dim, int64_t num_blocks,
                            int32_t max_blocks_per_seq, int32_t max_context_len,
                            float scale, int32_t partition_size,
                            int32_t q_dtype, int32_t cache_dtype,
                            void *workspace, size_t workspace_bytes,
                            void *stream, int32_t sliding_window);

/*
 * pa_decode_multi - paged attention of q_len new tokens per sequence (several
 * speculative tokens checked in one pass, "LLM推理引擎深度实战：…", §6.1; a chunk of a
 * long prompt, "大模型推理引擎优化：…", §4.1), causal within the new chunk.
 *
 * query and out are [num_seqs, q_len, num_heads, head_dim] (q_dtype);
 * context_lens count the q_len new tokens, which must already be in the cache
 * (pa_append_kv with num_seqs * q_len slots).  New token i of sequence b sits at
 * position L - q_len + i and attends to tokens 0 .. L - q_len + i (a zero row
 * when that range is empty).  q_len 1..4096; every other argument is as for
 * pa_decode, with the workspace size from pa_decode_multi_workspace_bytes.
 * Rows of (query, head) fill 16-row matrix-core tiles: a tile holds the heads of
 * one KV head and as many of a sequence's queries as fit.
 */
pa_status pa_decode_multi(void *out, const void *query,
                          const void *key_cache, const void *value_cache,
                          const float *k_scale, const float *v_scale,
                          const int32_t *block_tables, const int32_t *context_lens,
                          int32_t num_seqs, int32_t q_len, int32_t num_heads,
                          int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks,
                          int32_t max_blocks_per_seq, int32_t max_context_len,
                          float scale, int32_t partition_size,
                          int32_t q_dtype, int32_t cache_dtype,
                          void *workspace, size_t workspace_bytes,
                          void *stream);

/* pa_decode_multi_workspace_bytes - workspace pa_decode_multi needs ((size_t)-1: invalid). */
size_t pa_decode_multi_workspace_bytes(int32_t num_seqs, int32_t q_len, int32_t num_heads,
                                       int32_t num_kv_heads, int32_t head_dim,
                                       int32_t max_context_len, int32_t partition_size);

/* pa_decode_shared_prefix - paged decode for groups of sequences that share a prefix.
 *
 * Beam search and parallel sampling give several sequences the same prefix blocks,
 * shared through reference counts ("LLM推理引擎深度实战：从PagedAttention到分布式推理部署",
 * §2.2, copy-on-write; "大模型推理引擎优化：KV Cache 与连续批处理", §三 and §4.2).  The
 * result is exactly pa_decode's (up to rounding order): every sequence attends to its
 * own L_b tokens through its own page table.  What differs is the reading: sequences
 * g*group_size .. g*group_size + group_size - 1 form group g, and the first
 * prefix_blocks[g] page-table entries of group g are read once for all of its
 * sequences, whose query heads of one KV head fill the rows of one 16-row
 * matrix-core tile.
 *
 * prefix_blocks : int32 [num_seqs / group_size] on the device.  Caller contract: the
 *                 first prefix_blocks[g] entries of the tables of group g are equal
 *                 (values are clamped to [0, shortest sequence's block count]; a
 *                 wrong claim gives undefined results for that group, never an
 *                 out-of-pool access).
 * group_size    : 1..16, dividing num_seqs, with group_size * (num_heads /
 *                 num_kv_heads) <= 16; otherwise PA_ERR_SHAPE.
 * Always the balanced split (no partition_size); the workspace size comes from
 * pa_decode_shared_prefix_workspace_bytes.  Every other argument is as for pa_decode.
 * Errors (host checks only, before any launch): PA_ERR_SHAPE for a bad group size or
 * shape; PA_ERR_NULL for a missing pointer, prefix_blocks included; PA_ERR_ALIGN when
 * prefix_blocks is not 4-byte aligned (other buffers as for pa_decode);
 * PA_ERR_WORKSPACE; PA_ERR_DTYPE as for pa_decode; PA_ERR_HIP on a launch failure.
 */
pa_status pa_decode_shared_prefix(void *out, const void *query,
                                  const void *key_cache, const void *value_cache,
                                  const float *k_scale, const float *v_scale,
                                  const int32_t *block_tables, const int32_t *context_lens,
                                  const int32_t *prefix_blocks, int32_t group_size,
                                  int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int64_t num_blocks,
                                  int32_t max_blocks_per_seq, int32_t max_context_len,
                                  float scale, int32_t q_dtype, int32_t cache_dtype,
                                  void *workspace, size_t workspace_bytes, void *stream);

/* pa_decode_shared_prefix_workspace_bytes - workspace pa_decode_shared_prefix needs
 * ((size_t)-1: invalid shape). */
size_t pa_decode_shared_prefix_workspace_bytes(int32_t num_seqs, int32_t group_size,
                                               int32_t num_heads, int32_t num_kv_heads,
                                               int32_t head_dim, int32_t max_context_len);

/* pa_status_string - static, human-readable name of a status code. */
const char *pa_status_string(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_H */
