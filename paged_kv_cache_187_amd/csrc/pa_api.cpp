// C ABI entry points: host-side argument checks, launch configuration and
// dispatch to the gfx950 kernels.  Nothing here reads device memory or
// synchronises; see include/pagedattn.h for the contract.

#include "pagedattn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "pa_internal.h"

namespace {

constexpr int32_t kDefaultPartition = 512;       // tokens; 32 blocks
constexpr int32_t kMaxPartition = 1 << 20;
constexpr int64_t kMaxGrid = (int64_t)1 << 31;   // workgroups per launch

bool aligned(const void* ptr, uintptr_t a) { return ((uintptr_t)ptr & (a - 1)) == 0; }

bool is16(int32_t d) { return d == PA_F16 || d == PA_BF16; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Partition count of the grid; at least one so that L == 0 rows get written.
int64_t num_partitions(int32_t max_context_len, int32_t part) {
    const int64_t n = ceil_div(max_context_len, part);
    return n < 1 ? 1 : n;
}

pa_status from_hip(hipError_t e) { return e == hipSuccess ? PA_OK : PA_ERR_HIP; }

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

int32_t pa_decode_partition_size(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t max_context_len, int32_t partition_size) {
    if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || max_context_len < 0) return 0;
    if (partition_size != 0) {
        if (partition_size < 0 || partition_size % PA_BLOCK_SIZE != 0 || partition_size > kMaxPartition) return 0;
        return partition_size;
    }
    return kDefaultPartition;
}

size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t max_context_len, int32_t partition_size) {
    const int32_t part = pa_decode_partition_size(num_seqs, num_heads, num_kv_heads, head_dim, max_context_len,
                                                  partition_size);
    if (part <= 0) return (size_t)-1;
    const int64_t np = num_partitions(max_context_len, part);
    if (np <= 1) return 0;
    return (size_t)num_seqs * (size_t)num_heads * (size_t)np * (size_t)(head_dim + 2) * sizeof(float);
}

pa_status pa_decode(void* out, const void* query, const void* key_cache, const void* value_cache,
                    const float* k_scale, const float* v_scale, const int32_t* block_tables,
                    const int32_t* context_lens, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                    int32_t head_dim, int64_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
                    float scale, int32_t partition_size, int32_t q_dtype, int32_t cache_dtype, void* workspace,
                    size_t workspace_bytes, void* stream) {
    if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads != 0 ||
        num_blocks <= 0 || max_blocks_per_seq <= 0 || max_context_len < 0 || num_heads > 65536)
        return PA_ERR_SHAPE;
    if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
    if (!is16(q_dtype)) return PA_ERR_DTYPE;
    const bool fp8 = cache_dtype == PA_FP8_E4M3;
    if (!fp8 && cache_dtype != q_dtype) return PA_ERR_DTYPE;
    if (!std::isfinite(scale)) return PA_ERR_SHAPE;
    const int32_t part = pa_decode_partition_size(num_seqs, num_heads, num_kv_heads, head_dim, max_context_len,
                                                  partition_size);
    if (part <= 0) return PA_ERR_SHAPE;
    const size_t need = pa_decode_workspace_bytes(num_seqs, num_heads, num_kv_heads, head_dim, max_context_len,
                                                  partition_size);
    if (num_seqs == 0) return PA_OK;
    if (!out || !query || !key_cache || !value_cache || !block_tables || !context_lens) return PA_ERR_NULL;
    if (fp8 && (!k_scale || !v_scale)) return PA_ERR_NULL;
    if (need > 0 && (!workspace || workspace_bytes < need)) return PA_ERR_WORKSPACE;
    if (!aligned(out, 16) || !aligned(query, 16) || !aligned(key_cache, 16) || !aligned(value_cache, 16) ||
        !aligned(block_tables, 4) || !aligned(context_lens, 4) || (need > 0 && !aligned(workspace, 16)) ||
        (fp8 && (!aligned(k_scale, 4) || !aligned(v_scale, 4))))
        return PA_ERR_ALIGN;

    const int group = num_heads / num_kv_heads;
    const int hpw = pa::heads_per_workgroup(group);
    const int64_t np = num_partitions(max_context_len, part);
    const int64_t groups = num_heads / hpw;
    if (np * groups * num_seqs >= kMaxGrid) return PA_ERR_SHAPE;

    pa::DecodeParams p{};
    p.out = out;
    p.query = query;
    p.key_cache = key_cache;
    p.value_cache = value_cache;
    p.k_scale = fp8 ? k_scale : nullptr;
    p.v_scale = fp8 ? v_scale : nullptr;
    p.block_tables = block_tables;
    p.context_lens = context_lens;
    p.ws_acc = need > 0 ? (float*)workspace : nullptr;
    p.ws_ml = need > 0 ? (float*)workspace + (size_t)num_seqs * num_heads * np * head_dim : nullptr;
    p.num_blocks = num_blocks;
    p.B = num_seqs;
    p.Hq = num_heads;
    p.Hkv = num_kv_heads;
    p.max_blocks = max_blocks_per_seq;
    const int64_t table_tokens = (int64_t)max_blocks_per_seq * PA_BLOCK_SIZE;
    p.ctx_limit = (int32_t)(table_tokens < max_context_len ? table_tokens : max_context_len);
    p.NP = (int32_t)np;
    p.part_blocks = part / PA_BLOCK_SIZE;
    p.groups = (int32_t)groups;
    p.scale_log2 = scale * 1.4426950408889634f;
    return from_hip(pa::launch_decode(p, head_dim, q_dtype, cache_dtype, hpw, (hipStream_t)stream));
}

}  // extern "C"
