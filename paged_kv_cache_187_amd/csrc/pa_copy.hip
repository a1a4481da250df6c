// Whole-block copies for gfx950: copy-on-write and swap.
//
// Before a sequence writes into a block it shares with other sequences (its
// reference count is above one), the block manager gives it a private copy of
// that block ("大模型推理引擎优化：KV Cache 与连续批处理", §4.2; "LLM推理引擎深度实战：从
// PagedAttention到分布式推理部署", §2.2, copy-on-write for beam search and parallel
// sampling).  A preempted request's blocks are written out to CPU memory and read
// back when it resumes (same page, §3.2).  Both are the same operation: every
// (src, dst) pair copies the whole physical block src of the source K and V pools
// (and, for an FP8 cache, the block's 16 per-token scales of each) to block dst of
// the destination pools, bit for bit.  For copy-on-write both pools are the GPU
// pools; for a swap one of them is pinned host memory mapped into the GPU's
// address space, reached over PCIe by the same loads and stores.
//
// One workgroup per (pair, K-or-V, 16 KB chunk of the block), each lane moving
// four 16-byte vectors whose loads are all issued before the first store.

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kCopyThreads = 256;
constexpr int kCopyVecs = 4;                                  // 16-byte vectors per lane
constexpr int64_t kChunkVecs = (int64_t)kCopyThreads * kCopyVecs;   // 16 KB per workgroup

struct CopyPools {
    const uint4* src_k;
    const uint4* src_v;
    const float* src_ks;     // FP8 scales of the source pools (null: no scales)
    const float* src_vs;
    uint4* dst_k;
    uint4* dst_v;
    float* dst_ks;
    float* dst_vs;
    int64_t src_blocks, dst_blocks;
    int32_t same_pool;       // 1: src == dst pairs are skipped
};

__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(const CopyPools c,
                                                                  const int64_t* __restrict__ mapping,
                                                                  int64_t block_vecs) {
    const int64_t pair = blockIdx.x;
    const int64_t src = mapping[2 * pair];
    const int64_t dst = mapping[2 * pair + 1];
    if (src < 0 || src >= c.src_blocks || dst < 0 || dst >= c.dst_blocks || (c.same_pool && src == dst)) return;
    const bool is_v = blockIdx.y != 0;
    const uint4* from = (is_v ? c.src_v : c.src_k) + src * block_vecs;
    uint4* to = (is_v ? c.dst_v : c.dst_k) + dst * block_vecs;
    const int64_t base = (int64_t)blockIdx.z * kChunkVecs + threadIdx.x;
    // Each byte is moved once: streaming (non-temporal) loads and stores keep the copy from
    // displacing cached data of concurrent work.
    uint4 v[kCopyVecs];
#pragma unroll
    for (int i = 0; i < kCopyVecs; ++i) {
        const int64_t k = base + (int64_t)i * kCopyThreads;
        if (k < block_vecs) v[i] = load_stream(from + k);
    }
#pragma unroll
    for (int i = 0; i < kCopyVecs; ++i) {
        const int64_t k = base + (int64_t)i * kCopyThreads;
        if (k < block_vecs) store_stream(to + k, v[i]);
    }
    const float* sfrom = is_v ? c.src_vs : c.src_ks;
    float* sto = is_v ? c.dst_vs : c.dst_ks;
    if (sfrom != nullptr && blockIdx.z == 0 && threadIdx.x < kBlockSize)
        sto[dst * kBlockSize + threadIdx.x] = sfrom[src * kBlockSize + threadIdx.x];
}

}  // namespace

hipError_t launch_copy_blocks(const void* src_key, const void* src_value, const float* src_k_scale,
                              const float* src_v_scale, int64_t src_blocks, void* dst_key, void* dst_value,
                              float* dst_k_scale, float* dst_v_scale, int64_t dst_blocks, bool same_pool,
                              const int64_t* mapping, int64_t num_pairs, int64_t block_bytes, hipStream_t stream) {
    const int64_t block_vecs = block_bytes / 16;
    const int64_t chunks = (block_vecs + kChunkVecs - 1) / kChunkVecs;
    const CopyPools c{(const uint4*)src_key, (const uint4*)src_value, src_k_scale, src_v_scale,
                      (uint4*)dst_key,       (uint4*)dst_value,       dst_k_scale, dst_v_scale,
                      src_blocks,            dst_blocks,              same_pool ? 1 : 0};
    hipLaunchKernelGGL(copy_blocks_kernel, dim3((uint32_t)num_pairs, 2, (uint32_t)chunks), dim3(kCopyThreads), 0,
                       stream, c, mapping, block_vecs);
    return hipGetLastError();
}

}  // namespace pa
