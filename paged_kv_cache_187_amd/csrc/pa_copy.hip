// Copy-on-write block copy for gfx950.
//
// Before a sequence writes into a block it shares with other sequences (its
// reference count is above one), the block manager gives it a private copy of
// that block ("大模型推理引擎优化：KV Cache 与连续批处理", §4.2; "LLM推理引擎深度实战：从
// PagedAttention到分布式推理部署", §2.2, copy-on-write for beam search and parallel
// sampling).  This kernel makes those copies: every (src, dst) pair copies the
// whole physical block of the K pool and of the V pool, and for an FP8 cache the
// block's 16 per-token scales of each, bit for bit.
//
// The copy is bound by HBM bandwidth: one workgroup per (pair, K-or-V, 16 KB
// chunk of the block), each lane moving four 16-byte vectors whose loads are all
// issued before the first store.

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kCopyThreads = 256;
constexpr int kCopyVecs = 4;                                  // 16-byte vectors per lane
constexpr int64_t kChunkVecs = (int64_t)kCopyThreads * kCopyVecs;   // 16 KB per workgroup

__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(uint4* __restrict__ key_cache,
                                                                  uint4* __restrict__ value_cache,
                                                                  float* __restrict__ k_scale,
                                                                  float* __restrict__ v_scale,
                                                                  const int64_t* __restrict__ mapping,
                                                                  int64_t block_vecs, int64_t num_blocks) {
    const int64_t pair = blockIdx.x;
    const int64_t src = mapping[2 * pair];
    const int64_t dst = mapping[2 * pair + 1];
    if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks || src == dst) return;
    const bool is_v = blockIdx.y != 0;
    uint4* pool = is_v ? value_cache : key_cache;
    const uint4* from = pool + src * block_vecs;
    uint4* to = pool + dst * block_vecs;
    const int64_t base = (int64_t)blockIdx.z * kChunkVecs + threadIdx.x;
    uint4 v[kCopyVecs];
#pragma unroll
    for (int i = 0; i < kCopyVecs; ++i) {
        const int64_t k = base + (int64_t)i * kCopyThreads;
        if (k < block_vecs) v[i] = from[k];
    }
#pragma unroll
    for (int i = 0; i < kCopyVecs; ++i) {
        const int64_t k = base + (int64_t)i * kCopyThreads;
        if (k < block_vecs) to[k] = v[i];
    }
    float* scales = is_v ? v_scale : k_scale;
    if (scales != nullptr && blockIdx.z == 0 && threadIdx.x < kBlockSize)
        scales[dst * kBlockSize + threadIdx.x] = scales[src * kBlockSize + threadIdx.x];
}

}  // namespace

hipError_t launch_copy_blocks(void* key_cache, void* value_cache, float* k_scale, float* v_scale,
                              const int64_t* mapping, int64_t num_pairs, int64_t block_bytes, int64_t num_blocks,
                              hipStream_t stream) {
    const int64_t block_vecs = block_bytes / 16;
    const int64_t chunks = (block_vecs + kChunkVecs - 1) / kChunkVecs;
    hipLaunchKernelGGL(copy_blocks_kernel, dim3((uint32_t)num_pairs, 2, (uint32_t)chunks), dim3(kCopyThreads), 0,
                       stream, (uint4*)key_cache, (uint4*)value_cache, k_scale, v_scale, mapping, block_vecs,
                       num_blocks);
    return hipGetLastError();
}

}  // namespace pa
