// Host-side launchers behind the C ABI.  Arguments are already validated by
// the entry points in pa_api.cpp.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// Kind codes used between the C ABI and the launchers (same values as pa_dtype).
enum Kind { kF16 = 0, kBF16 = 1, kFP8 = 2 };

struct DecodeParams {
    void* out;                 // [B, Hq, D] q dtype
    const void* query;         // [B, Hq, D] q dtype
    const void* key_cache;     // [num_blocks, 16, Hkv, D] cache dtype
    const void* value_cache;
    const float* k_scale;      // [num_blocks, 16] (FP8 cache)
    const float* v_scale;
    const int32_t* block_tables;  // [B, max_blocks]
    const int32_t* context_lens;  // [B]
    float* ws_acc;             // [slots, HPW, D] partial V sums
    float* ws_ml;              // [slots, HPW, 2] partial (max, sum of exponentials)
    int64_t num_blocks;
    int32_t B, Hq, Hkv, max_blocks, ctx_limit;  // ctx_limit = min(max_context_len, 16 * max_blocks)
    int32_t balanced;          // 1: equal (sequence, block) ranges per team of `groups` waves
    int32_t NP;                // fixed split: partitions per sequence in the grid
    int32_t part_blocks;       // fixed split: partition length in 16-token blocks
    int32_t groups;            // work units per sequence = (Hq / hpw) head groups x qgroups query groups
    int32_t qlen;              // new tokens (queries) per sequence: 1 for decode
    int32_t qpw;               // queries per unit (matrix-core path): rows = qpw x hpw <= 16
    int32_t qgroups;           // query groups per head group = ceil(qlen / qpw)
    int32_t rows;              // rows per unit = qpw x hpw (partial-result rows per slot)
    int32_t hpw;               // query heads per wave (all share one KV head)
    int32_t mfma;              // 1: matrix-core path (hpw <= 16 rows of a 16x16 tile)
    int32_t num_waves;         // waves in the grid
    int32_t teams;             // balanced split: teams of `groups` waves, one range of blocks each
    int32_t window;            // sliding window in tokens (0: attend to the whole context)
    float scale_log2;          // softmax scale * log2(e)
    // Shared-prefix groups (matrix-core path, balanced split): sequences g*sgroup ..
    // g*sgroup + sgroup - 1 form group g and share their first prefix_blocks[g] page-table
    // entries; a unit holds the group's sequences as tile rows.  sgroup == 0: no groups.
    int32_t sgroup;
    const int32_t* prefix_blocks;  // [B / sgroup]
    // Fused append + decode (16-bit caches): the new token of sequence b (position L_b - 1) has
    // K/V rows new_key[b], new_value[b] ([B, Hkv, D], the cache dtype), written into its slot by
    // the decode kernel itself.  Null for the plain decode.
    const void* new_key;
    const void* new_value;
};

hipError_t launch_append_copy(const void* key, const void* value, void* key_cache, void* value_cache,
                              const int64_t* slots, int64_t num_tokens, int32_t row_bytes,
                              int64_t num_slots, hipStream_t stream);

hipError_t launch_append_fp8(const void* key, const void* value, void* key_cache, void* value_cache,
                             float* k_scale, float* v_scale, const int64_t* slots, int64_t num_tokens,
                             int32_t row_elems, int64_t num_slots, int src_kind, hipStream_t stream);

// The quantising append of each sequence's new token at position L - 1 (L = context_lens[b]
// clamped to [0, ctx_limit]; nothing for L == 0), the slot taken from the page table.
hipError_t launch_append_fp8_at_lengths(const void* key, const void* value, void* key_cache, void* value_cache,
                                        float* k_scale, float* v_scale, const int32_t* block_tables,
                                        const int32_t* context_lens, int32_t num_seqs, int32_t max_blocks,
                                        int32_t ctx_limit, int32_t row_elems, int64_t num_slots, int src_kind,
                                        hipStream_t stream);

// Whole-block copies from block src of the source pools to block dst of the destination
// pools for (src, dst) pairs (FP8 scales too when the scale pointers are not null);
// block_bytes is the bytes of one block of one pool.  same_pool: the pools are the same
// buffers (pairs with src == dst are skipped).
hipError_t launch_copy_blocks(const void* src_key, const void* src_value, const float* src_k_scale,
                              const float* src_v_scale, int64_t src_blocks, void* dst_key, void* dst_value,
                              float* dst_k_scale, float* dst_v_scale, int64_t dst_blocks, bool same_pool,
                              const int64_t* mapping, int64_t num_pairs, int64_t block_bytes, hipStream_t stream);

// Query heads of one KV head handled together by one wave, and whether that
// wave uses the matrix cores.
struct HeadGrouping {
    int hpw;
    bool mfma;
};
HeadGrouping head_grouping(int group);          // one query per sequence
HeadGrouping multi_query_grouping(int group);  // several queries per sequence

hipError_t launch_decode(const DecodeParams& p, int head_dim, int q_kind, int cache_kind, hipStream_t stream);
// The same decode with the append of each sequence's new token fused in (new_key/new_value set).
hipError_t launch_decode_append(const DecodeParams& p, int head_dim, int q_kind, int cache_kind,
                                hipStream_t stream);

// Device address of the fixed decode scratch on the current device (resolved once per
// device); used only by pa_decode_noalloc.
hipError_t scratch_address(void** out);

}  // namespace pa
