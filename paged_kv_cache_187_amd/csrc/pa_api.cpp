// C ABI entry points: host-side argument checks, launch configuration and
// dispatch to the gfx950 kernels.  Nothing here reads device memory or
// synchronises; see include/pagedattn.h for the contract.

#include "pagedattn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <algorithm>
#include <cstdint>

#include "pa_internal.h"

namespace {

constexpr int32_t kMaxPartition = 1 << 20;
constexpr int64_t kMaxWork = ((int64_t)1 << 30);  // waves, or (head group, block) pairs, per launch
// Waves of the balanced split.  One wave per SIMD keeps the memory system saturated for
// 16-bit caches (the matrix-core path streams two blocks per ring entry).  An FP8 block
// carries half the bytes for about the same work per block, so FP8 caches run two waves
// per SIMD, one wave's conversions and matrix products overlapping the other's loads.
// Shared-prefix groups stay at 1024 waves: their ranges are at least 16 positions long, so
// more waves would leave teams idle and crowd the working ones onto half of the CUs.
// Workspace queries size for the larger count (an upper bound).
constexpr int64_t kBalancedWaves = 1024;       // 4 per CU
constexpr int64_t kBalancedWavesFp8 = 2048;    // 8 per CU
constexpr int32_t kMaxQueries = 4096;               // new tokens per sequence in one multi-query call

// Launch shape shared by pa_decode and pa_decode_workspace_bytes.
struct Plan {
    bool ok;
    bool balanced;
    int64_t part;        // fixed split: partition tokens
    int64_t np;          // fixed split: partitions per sequence
    int64_t hpw;         // heads per wave
    int64_t qpw;         // queries per wave (rows = qpw x hpw)
    int64_t qgroups;     // query groups per head group
    bool mfma;           // matrix-core path
    int64_t groups;      // head groups per sequence
    int64_t waves;       // waves in the grid
    int64_t teams;       // balanced split: teams of `groups` waves (one per head group)
    int64_t slots;       // workspace slots (each HPW heads x (D + 2) floats)
};

// seq_group > 0: shared-prefix groups of seq_group consecutive sequences, each unit holding
// the group's sequences times the query heads of one KV head as rows of a 16-row tile.
Plan make_plan(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
               int32_t max_context_len, int32_t partition_size, int32_t q_len = 1, int32_t seq_group = 0,
               bool fp8 = true) {
    Plan pl{};
    if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads != 0 || head_dim <= 0 ||
        max_context_len < 0 || partition_size < 0 || partition_size % PA_BLOCK_SIZE != 0 ||
        partition_size > kMaxPartition || q_len < 1 || q_len > kMaxQueries || seq_group < 0)
        return pl;
    const int32_t group = num_heads / num_kv_heads;
    if (seq_group > 0 &&
        (q_len != 1 || partition_size != 0 || num_seqs % seq_group != 0 || (int64_t)seq_group * group > 16))
        return pl;
    const pa::HeadGrouping hg = seq_group > 0 ? pa::HeadGrouping{group, true}
                                : q_len == 1  ? pa::head_grouping(group)
                                              : pa::multi_query_grouping(group);
    pl.hpw = hg.hpw;
    pl.mfma = hg.mfma;
    pl.qpw = seq_group > 0 ? seq_group : q_len == 1 ? 1 : std::min<int64_t>(q_len, 16 / pl.hpw);
    pl.qgroups = seq_group > 0 ? 1 : (q_len + pl.qpw - 1) / pl.qpw;
    pl.groups = num_heads / pl.hpw * pl.qgroups;
    const int64_t entries = seq_group > 0 ? num_seqs / seq_group : num_seqs;
    const int64_t seq_groups = entries * pl.groups;
    const int64_t max_blocks = (max_context_len + PA_BLOCK_SIZE - 1) / PA_BLOCK_SIZE *
                               (seq_group > 0 ? seq_group : 1);   // per entry
    if (seq_groups * (max_blocks > 0 ? max_blocks : 1) >= kMaxWork) return pl;
    pl.balanced = partition_size == 0;
    if (pl.balanced) {
        // Teams of one wave per head group share a range of (sequence, block) positions:
        // about balanced_waves waves, at most one team per block and at least one team.
        const int64_t blocks = entries * max_blocks;   // upper bound of (entry, block) positions
        const int64_t balanced_waves = fp8 && seq_group == 0 ? kBalancedWavesFp8 : kBalancedWaves;
        int64_t teams = balanced_waves / pl.groups;
        if (teams > blocks) teams = blocks;
        if (teams < 1) teams = 1;
        pl.teams = teams;
        pl.waves = teams * pl.groups;
        // a partial goes to slot hg * (teams + entries) + range + entry
        pl.slots = pl.groups * (teams + entries);
    } else {
        pl.part = partition_size;
        pl.np = (max_context_len + partition_size - 1) / partition_size;
        if (pl.np < 1) pl.np = 1;
        pl.waves = pl.np * seq_groups;
        pl.slots = pl.np > 1 ? pl.np * seq_groups : 0;
    }
    pl.ok = pl.waves < kMaxWork;
    return pl;
}

size_t workspace_size(const Plan& pl, int32_t head_dim) {
    return (size_t)pl.slots * (size_t)(pl.hpw * pl.qpw) * (size_t)(head_dim + 2) * sizeof(float);
}

bool aligned(const void* ptr, uintptr_t a) { return ((uintptr_t)ptr & (a - 1)) == 0; }

bool is16(int32_t d) { return d == PA_F16 || d == PA_BF16; }

pa_status from_hip(hipError_t e) { return e == hipSuccess ? PA_OK : PA_ERR_HIP; }

// Host checks shared by the block copies (one pool's pointers and sizes).
pa_status check_copy(const void* key, const void* value, const float* k_scale, const float* v_scale,
                     const int64_t* mapping, int64_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                     int64_t num_blocks, int32_t cache_dtype) {
    if (num_pairs < 0 || num_pairs > ((int64_t)1 << 31) - 1 || num_kv_heads <= 0 || num_kv_heads > 4096 ||
        num_blocks <= 0)
        return PA_ERR_SHAPE;
    if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
    const bool fp8 = cache_dtype == PA_FP8_E4M3;
    if (!fp8 && !is16(cache_dtype)) return PA_ERR_DTYPE;
    if (num_pairs == 0) return PA_OK;
    if (!key || !value || !mapping) return PA_ERR_NULL;
    if (fp8 && (!k_scale || !v_scale)) return PA_ERR_NULL;
    if (!aligned(key, 16) || !aligned(value, 16) || !aligned(mapping, 8) ||
        (fp8 && (!aligned(k_scale, 4) || !aligned(v_scale, 4))))
        return PA_ERR_ALIGN;
    return PA_OK;
}

// True when the GPU reaches `p` at the same address: device memory, or host memory
// pinned and mapped into the GPU's address space.  A failed query leaves no error
// behind for the launch check that follows.
bool gpu_addressable(const void* p) {
    if (p == nullptr) return true;
    hipPointerAttribute_t a{};
    if (hipPointerGetAttributes(&a, p) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    return a.devicePointer == p;
}

int64_t block_bytes(int32_t num_kv_heads, int32_t head_dim, bool fp8) {
    return (int64_t)PA_BLOCK_SIZE * num_kv_heads * head_dim * (fp8 ? 1 : 2);
}

}  // namespace

namespace {

pa_status decode_impl(void* out, const void* query, const void* key_cache, const void* value_cache,
                    const float* k_scale, const float* v_scale, const int32_t* block_tables,
                    const int32_t* context_lens, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                    int32_t head_dim, int64_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
                    float scale, int32_t partition_size, int32_t q_dtype, int32_t cache_dtype, void* workspace,
                    size_t workspace_bytes, void* stream, int32_t window, int32_t q_len,
                    int32_t seq_group = 0, const int32_t* prefix_blocks = nullptr, bool use_scratch = false,
                    const void* new_key = nullptr, const void* new_value = nullptr) {
    if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads != 0 ||
        num_blocks <= 0 || max_blocks_per_seq <= 0 || max_context_len < 0 || num_heads > 65536)
        return PA_ERR_SHAPE;
    if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
    if (!is16(q_dtype)) return PA_ERR_DTYPE;
    const bool fp8 = cache_dtype == PA_FP8_E4M3;
    if (!fp8 && cache_dtype != q_dtype) return PA_ERR_DTYPE;
    if (!std::isfinite(scale) || window < 0) return PA_ERR_SHAPE;
    const Plan pl = make_plan(num_seqs, num_heads, num_kv_heads, head_dim, max_context_len, partition_size, q_len,
                              seq_group, fp8);
    if (!pl.ok) return PA_ERR_SHAPE;
    const size_t need = workspace_size(pl, head_dim);
    if (use_scratch && need > PA_NOALLOC_SCRATCH_BYTES) return PA_ERR_SCRATCH;
    if (num_seqs == 0) return PA_OK;
    if (!out || !query || !key_cache || !value_cache || !block_tables || !context_lens) return PA_ERR_NULL;
    if (seq_group > 0 && !prefix_blocks) return PA_ERR_NULL;
    if (fp8 && (!k_scale || !v_scale)) return PA_ERR_NULL;
    const bool fused = new_key != nullptr || new_value != nullptr;
    if (fused && (!new_key || !new_value)) return PA_ERR_NULL;
    if (fused && (!aligned(new_key, 16) || !aligned(new_value, 16))) return PA_ERR_ALIGN;
    if (use_scratch) {
        workspace = nullptr;
        workspace_bytes = 0;
    }
    if (!use_scratch && need > 0 && (!workspace || workspace_bytes < need)) return PA_ERR_WORKSPACE;
    if (!aligned(out, 16) || !aligned(query, 16) || !aligned(key_cache, 16) || !aligned(value_cache, 16) ||
        !aligned(block_tables, 4) || !aligned(context_lens, 4) || (need > 0 && !aligned(workspace, 16)) ||
        (seq_group > 0 && !aligned(prefix_blocks, 4)) ||
        (fp8 && (!aligned(k_scale, 4) || !aligned(v_scale, 4))))
        return PA_ERR_ALIGN;
    if (use_scratch && need > 0) {
        // every host check has passed: only now touch the device
        if (pa::scratch_address(&workspace) != hipSuccess) return PA_ERR_HIP;
        workspace_bytes = PA_NOALLOC_SCRATCH_BYTES;
    }

    pa::DecodeParams p{};
    p.out = out;
    p.query = query;
    p.key_cache = key_cache;
    p.value_cache = value_cache;
    p.k_scale = fp8 ? k_scale : nullptr;
    p.v_scale = fp8 ? v_scale : nullptr;
    p.block_tables = block_tables;
    p.context_lens = context_lens;
    if (need > 0) {
        p.ws_acc = (float*)workspace;
        p.ws_ml = p.ws_acc + (size_t)pl.slots * pl.hpw * pl.qpw * head_dim;
    }
    p.num_blocks = num_blocks;
    p.B = num_seqs;
    p.Hq = num_heads;
    p.Hkv = num_kv_heads;
    p.max_blocks = max_blocks_per_seq;
    const int64_t table_tokens = (int64_t)max_blocks_per_seq * PA_BLOCK_SIZE;
    p.ctx_limit = (int32_t)(table_tokens < max_context_len ? table_tokens : max_context_len);
    p.balanced = pl.balanced ? 1 : 0;
    p.NP = (int32_t)pl.np;
    p.part_blocks = (int32_t)(pl.part / PA_BLOCK_SIZE);
    p.groups = (int32_t)pl.groups;
    p.hpw = (int32_t)pl.hpw;
    p.qlen = q_len;
    p.qpw = (int32_t)pl.qpw;
    p.qgroups = (int32_t)pl.qgroups;
    p.rows = (int32_t)(pl.qpw * pl.hpw);
    p.mfma = pl.mfma ? 1 : 0;
    p.num_waves = (int32_t)pl.waves;
    p.teams = (int32_t)pl.teams;
    p.window = window;
    p.scale_log2 = scale * 1.4426950408889634f;
    p.sgroup = seq_group;
    p.prefix_blocks = seq_group > 0 ? prefix_blocks : nullptr;
    if (fused && fp8) {
        // an FP8 cache's quantising append runs first, as its own kernel, at the slots the page
        // tables give; then the plain decode
        const hipError_t e = pa::launch_append_fp8_at_lengths(
            new_key, new_value, (void*)key_cache, (void*)value_cache, (float*)k_scale, (float*)v_scale, block_tables,
            context_lens, num_seqs, max_blocks_per_seq, p.ctx_limit, num_kv_heads * head_dim,
            num_blocks * PA_BLOCK_SIZE, q_dtype, (hipStream_t)stream);
        if (e != hipSuccess) return PA_ERR_HIP;
        return from_hip(pa::launch_decode(p, head_dim, q_dtype, cache_dtype, (hipStream_t)stream));
    }
    p.new_key = new_key;
    p.new_value = new_value;
    if (fused) return from_hip(pa::launch_decode_append(p, head_dim, q_dtype, cache_dtype, (hipStream_t)stream));
    return from_hip(pa::launch_decode(p, head_dim, q_dtype, cache_dtype, (hipStream_t)stream));
}

}  // namespace

extern "C" {

const char* pa_status_string(int32_t status) {
    switch (status) {
        case PA_OK: return "PA_OK";
        case PA_ERR_NULL: return "PA_ERR_NULL: a required pointer is NULL";
        case PA_ERR_SHAPE: return "PA_ERR_SHAPE: a size is out of range or inconsistent";
        case PA_ERR_DTYPE: return "PA_ERR_DTYPE: unsupported dtype or dtype combination";
        case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED: head_dim must be 64 or 128";
        case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE: workspace missing or too small";
        case PA_ERR_HIP: return "PA_ERR_HIP: the HIP runtime reported an error";
        case PA_ERR_ALIGN: return "PA_ERR_ALIGN: a buffer is not 16-byte aligned";
        case PA_ERR_ADDRESS: return "PA_ERR_ADDRESS: a buffer is not addressable by the GPU";
        case PA_ERR_SCRATCH:
            return "PA_ERR_SCRATCH: the call needs more workspace than the fixed scratch of pa_decode_noalloc "
                   "(PA_NOALLOC_SCRATCH_BYTES); use pa_decode with a workspace";
        default: return "unknown pa_status";
    }
}

pa_status pa_append_kv(const void* key, const void* value, void* key_cache, void* value_cache, float* k_scale,
                       float* v_scale, const int64_t* slot_mapping, int64_t num_tokens, int32_t num_kv_heads,
                       int32_t head_dim, int64_t num_blocks, int32_t src_dtype, int32_t cache_dtype,
                       void* stream) {
    if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks <= 0 || num_tokens > ((int64_t)1 << 31) - 1 ||
        num_kv_heads > 4096)
        return PA_ERR_SHAPE;
    if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
    if (!is16(src_dtype)) return PA_ERR_DTYPE;
    const bool fp8 = cache_dtype == PA_FP8_E4M3;
    if (!fp8 && cache_dtype != src_dtype) return PA_ERR_DTYPE;
    if (num_tokens == 0) return PA_OK;
    if (!key || !value || !key_cache || !value_cache || !slot_mapping) return PA_ERR_NULL;
    if (fp8 && (!k_scale || !v_scale)) return PA_ERR_NULL;
    if (!aligned(key, 16) || !aligned(value, 16) || !aligned(key_cache, 16) || !aligned(value_cache, 16) ||
        !aligned(slot_mapping, 8) || (fp8 && (!aligned(k_scale, 4) || !aligned(v_scale, 4))))
        return PA_ERR_ALIGN;
    const int64_t num_slots = num_blocks * PA_BLOCK_SIZE;
    const int32_t row_elems = num_kv_heads * head_dim;
    hipStream_t s = (hipStream_t)stream;
    if (!fp8) {
        return from_hip(pa::launch_append_copy(key, value, key_cache, value_cache, slot_mapping, num_tokens,
                                               row_elems * 2, num_slots, s));
    }
    return from_hip(pa::launch_append_fp8(key, value, key_cache, value_cache, k_scale, v_scale, slot_mapping,
                                          num_tokens, row_elems, num_slots, src_dtype, s));
}

pa_status pa_copy_blocks(void* key_cache, void* value_cache, float* k_scale, float* v_scale,
                         const int64_t* block_mapping, int64_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                         int64_t num_blocks, int32_t cache_dtype, void* stream) {
    const pa_status st = check_copy(key_cache, value_cache, k_scale, v_scale, block_mapping, num_pairs, num_kv_heads,
                                    head_dim, num_blocks, cache_dtype);
    if (st != PA_OK || num_pairs == 0) return st;
    const bool fp8 = cache_dtype == PA_FP8_E4M3;
    return from_hip(pa::launch_copy_blocks(key_cache, value_cache, fp8 ? k_scale : nullptr, fp8 ? v_scale : nullptr,
                                           num_blocks, key_cache, value_cache, fp8 ? k_scale : nullptr,
                                           fp8 ? v_scale : nullptr, num_blocks, true, block_mapping, num_pairs,
                                           block_bytes(num_kv_heads, head_dim, fp8), (hipStream_t)stream));
}

pa_status pa_swap_blocks(const void* src_key, const void* src_value, const float* src_k_scale,
                         const float* src_v_scale, int64_t src_num_blocks, void* dst_key, void* dst_value,
                         float* dst_k_scale, float* dst_v_scale, int64_t dst_num_blocks,
                         const int64_t* block_mapping, int64_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                         int32_t cache_dtype, void* stream) {
    pa_status st = check_copy(src_key, src_value, src_k_scale, src_v_scale, block_mapping, num_pairs, num_kv_heads,
                              head_dim, src_num_blocks, cache_dtype);
    if (st == PA_OK)
        st = check_copy(dst_key, dst_value, dst_k_scale, dst_v_scale, block_mapping, num_pairs, num_kv_heads,
                        head_dim, dst_num_blocks, cache_dtype);
    if (st != PA_OK || num_pairs == 0) return st;
    const bool fp8 = cache_dtype == PA_FP8_E4M3;
    const void* bufs[] = {src_key, src_value, dst_key, dst_value, block_mapping,
                          fp8 ? src_k_scale : nullptr, fp8 ? src_v_scale : nullptr,
                          fp8 ? dst_k_scale : nullptr, fp8 ? dst_v_scale : nullptr};
    for (const void* b : bufs)
        if (!gpu_addressable(b)) return PA_ERR_ADDRESS;
    return from_hip(pa::launch_copy_blocks(src_key, src_value, fp8 ? src_k_scale : nullptr,
                                           fp8 ? src_v_scale : nullptr, src_num_blocks, dst_key, dst_value,
                                           fp8 ? dst_k_scale : nullptr, fp8 ? dst_v_scale : nullptr, dst_num_blocks,
                                           false, block_mapping, num_pairs, block_bytes(num_kv_heads, head_dim, fp8),
                                           (hipStream_t)stream));
}

int32_t pa_decode_partition_size(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t max_context_len, int32_t partition_size) {
    const Plan pl = make_plan(num_seqs, num_heads, num_kv_heads, head_dim, max_context_len, partition_size);
    if (!pl.ok) return -1;
    return pl.balanced ? 0 : (int32_t)pl.part;
}

size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t max_context_len, int32_t partition_size) {
    const Plan pl = make_plan(num_seqs, num_heads, num_kv_heads, head_dim, max_context_len, partition_size);
    if (!pl.ok) return (size_t)-1;
    return workspace_size(pl, head_dim);
}

pa_status pa_decode(void* out, const void* query, const void* key_cache, const void* value_cache,
                    const float* k_scale, const float* v_scale, const int32_t* block_tables,
                    const int32_t* context_lens, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                    int32_t head_dim, int64_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
                    float scale, int32_t partition_size, int32_t q_dtype, int32_t cache_dtype, void* workspace,
                    size_t workspace_bytes, void* stream) {
    return decode_impl(out, query, key_cache, value_cache, k_scale, v_scale, block_tables, context_lens, num_seqs,
                       num_heads, num_kv_heads, head_dim, num_blocks, max_blocks_per_seq, max_context_len, scale,
                       partition_size, q_dtype, cache_dtype, workspace, workspace_bytes, stream, 0, 1);
}

pa_status pa_decode_append(void* out, const void* query, const void* key_new, const void* value_new,
                           void* key_cache, void* value_cache, float* k_scale, float* v_scale,
                           const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                           int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks,
                           int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                           int32_t partition_size, int32_t q_dtype, int32_t cache_dtype, void* workspace,
                           size_t workspace_bytes, void* stream) {
    if (!key_new || !value_new) return PA_ERR_NULL;
    return decode_impl(out, query, key_cache, value_cache, k_scale, v_scale, block_tables, context_lens, num_seqs,
                       num_heads, num_kv_heads, head_dim, num_blocks, max_blocks_per_seq, max_context_len, scale,
                       partition_size, q_dtype, cache_dtype, workspace, workspace_bytes, stream, 0, 1, 0, nullptr,
                       false, key_new, value_new);
}

pa_status pa_decode_noalloc(void* out, const void* query, const void* key_cache, const void* value_cache,
                            const float* k_scale, const float* v_scale, const int32_t* block_tables,
                            const int32_t* context_lens, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                            int32_t head_dim, int64_t num_blocks, int32_t max_blocks_per_seq,
                            int32_t max_context_len, float scale, int32_t partition_size, int32_t q_dtype,
                            int32_t cache_dtype, void* stream) {
    return decode_impl(out, query, key_cache, value_cache, k_scale, v_scale, block_tables, context_lens, num_seqs,
                       num_heads, num_kv_heads, head_dim, num_blocks, max_blocks_per_seq, max_context_len, scale,
                       partition_size, q_dtype, cache_dtype, nullptr, 0, stream, 0, 1, 0, nullptr, true);
}

pa_status pa_decode_sliding(void* out, const void* query, const void* key_cache, const void* value_cache,
                            const float* k_scale, const float* v_scale, const int32_t* block_tables,
                            const int32_t* context_lens, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                            int32_t head_dim, int64_t num_blocks, int32_t max_blocks_per_seq,
                            int32_t max_context_len, float scale, int32_t partition_size, int32_t q_dtype,
                            int32_t cache_dtype, void* workspace, size_t workspace_bytes, void* stream,
                            int32_t sliding_window) {
    return decode_impl(out, query, key_cache, value_cache, k_scale, v_scale, block_tables, context_lens, num_seqs,
                       num_heads, num_kv_heads, head_dim, num_blocks, max_blocks_per_seq, max_context_len, scale,
                       partition_size, q_dtype, cache_dtype, workspace, workspace_bytes, stream, sliding_window,
                       1);
}

pa_status pa_decode_multi(void* out, const void* query, const void* key_cache, const void* value_cache,
                          const float* k_scale, const float* v_scale, const int32_t* block_tables,
                          const int32_t* context_lens, int32_t num_seqs, int32_t q_len, int32_t num_heads,
                          int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks, int32_t max_blocks_per_seq,
                          int32_t max_context_len, float scale, int32_t partition_size, int32_t q_dtype,
                          int32_t cache_dtype, void* workspace, size_t workspace_bytes, void* stream) {
    if (q_len < 1 || q_len > kMaxQueries) return PA_ERR_SHAPE;
    return decode_impl(out, query, key_cache, value_cache, k_scale, v_scale, block_tables, context_lens, num_seqs,
                       num_heads, num_kv_heads, head_dim, num_blocks, max_blocks_per_seq, max_context_len, scale,
                       partition_size, q_dtype, cache_dtype, workspace, workspace_bytes, stream, 0, q_len);
}

pa_status pa_decode_shared_prefix(void* out, const void* query, const void* key_cache, const void* value_cache,
                                  const float* k_scale, const float* v_scale, const int32_t* block_tables,
                                  const int32_t* context_lens, const int32_t* prefix_blocks, int32_t group_size,
                                  int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                  int64_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
                                  float scale, int32_t q_dtype, int32_t cache_dtype, void* workspace,
                                  size_t workspace_bytes, void* stream) {
    if (group_size < 1 || group_size > 16) return PA_ERR_SHAPE;
    return decode_impl(out, query, key_cache, value_cache, k_scale, v_scale, block_tables, context_lens, num_seqs,
                       num_heads, num_kv_heads, head_dim, num_blocks, max_blocks_per_seq, max_context_len, scale, 0,
                       q_dtype, cache_dtype, workspace, workspace_bytes, stream, 0, 1, group_size, prefix_blocks);
}

size_t pa_decode_shared_prefix_workspace_bytes(int32_t num_seqs, int32_t group_size, int32_t num_heads,
                                               int32_t num_kv_heads, int32_t head_dim, int32_t max_context_len) {
    if (group_size < 1 || group_size > 16) return (size_t)-1;
    const Plan pl = make_plan(num_seqs, num_heads, num_kv_heads, head_dim, max_context_len, 0, 1, group_size);
    if (!pl.ok) return (size_t)-1;
    return workspace_size(pl, head_dim);
}

size_t pa_decode_multi_workspace_bytes(int32_t num_seqs, int32_t q_len, int32_t num_heads, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t max_context_len, int32_t partition_size) {
    const Plan pl = make_plan(num_seqs, num_heads, num_kv_heads, head_dim, max_context_len, partition_size, q_len);
    if (!pl.ok) return (size_t)-1;
    return workspace_size(pl, head_dim);
}

}  // extern "C"
