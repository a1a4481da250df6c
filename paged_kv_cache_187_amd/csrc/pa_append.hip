// Slot-mapped KV append (reshape_and_cache) for gfx950.
//
// Each decode step writes the new token's K and V rows into the slot the
// block manager assigned to it: block slot / 16, offset slot % 16
// ("大模型推理引擎优化：KV Cache 与连续批处理", §2.1-§2.2).  The FP8 variant quantises the
// token's K (and separately V) with one float32 scale per token
// ("LLM推理引擎深度实战：从PagedAttention到分布式推理部署", §5.3).
//
// One workgroup per (token, K-or-V): the rows are a few KB, so the work is
// launch-bound and the layout only has to keep the 16-byte accesses
// contiguous.

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

// Bit-exact copy of one token's [Hkv, D] row, 16 bytes per lane.
__global__ __launch_bounds__(256) void append_copy_kernel(const uint4* __restrict__ key,
                                                          const uint4* __restrict__ value,
                                                          uint4* __restrict__ key_cache,
                                                          uint4* __restrict__ value_cache,
                                                          const int64_t* __restrict__ slots,
                                                          int32_t row_vec, int64_t num_slots) {
    const int64_t t = blockIdx.x;
    const int64_t slot = slots[t];
    if (slot < 0 || slot >= num_slots) return;
    const uint4* src = (blockIdx.y == 0 ? key : value) + t * row_vec;
    uint4* dst = (blockIdx.y == 0 ? key_cache : value_cache) + slot * row_vec;
    for (int i = threadIdx.x; i < row_vec; i += blockDim.x) dst[i] = src[i];
}

// Where token t goes: slots[t], or, without a slot list, the position L - 1 of sequence t
// (L its length clamped to [0, ctx_limit]) through its page table; -1 for none.
struct SlotSource {
    const int64_t* slots;
    const int32_t* tables;
    const int32_t* lens;
    int32_t max_blocks, ctx_limit;

    __device__ int64_t slot(int64_t t) const {
        if (slots) return slots[t];
        int L = lens[t];
        L = L < 0 ? 0 : (L > ctx_limit ? ctx_limit : L);
        if (L == 0) return -1;
        const int32_t phys = tables[t * max_blocks + (L - 1) / kBlockSize];
        return phys < 0 ? -1 : (int64_t)phys * kBlockSize + (L - 1) % kBlockSize;
    }
};

// Per-token E4M3 quantisation of one token's [Hkv, D] row.  Eight source
// elements (16 bytes) per lane per step; codes are stored 8 bytes at a time.
template <typename SRC>
__global__ __launch_bounds__(256) void append_fp8_kernel(const uint4* __restrict__ key,
                                                         const uint4* __restrict__ value,
                                                         uint2* __restrict__ key_cache,
                                                         uint2* __restrict__ value_cache,
                                                         float* __restrict__ k_scale,
                                                         float* __restrict__ v_scale,
                                                         const SlotSource src_slots,
                                                         int32_t row_chunks, int64_t num_slots) {
    __shared__ float wave_max[256 / kWave];
    const int64_t t = blockIdx.x;
    const int64_t slot = src_slots.slot(t);
    if (slot < 0 || slot >= num_slots) return;
    const bool is_v = blockIdx.y != 0;
    const uint4* src = (is_v ? value : key) + t * row_chunks;
    uint2* dst = (is_v ? value_cache : key_cache) + slot * row_chunks;

    // amax over the whole token row (exact: max of magnitudes).
    float amax = 0.0f;
    for (int i = threadIdx.x; i < row_chunks; i += blockDim.x) {
        const uint4 w = src[i];
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float2_t f = unpack2(SRC{}, ws[k]);
            amax = __builtin_fmaxf(amax, __builtin_fmaxf(__builtin_fabsf(f.x), __builtin_fabsf(f.y)));
        }
    }
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) amax = __builtin_fmaxf(amax, __shfl_xor(amax, off));
    const int wave = threadIdx.x / kWave;
    if ((threadIdx.x & (kWave - 1)) == 0) wave_max[wave] = amax;
    __syncthreads();
    amax = wave_max[0];
    for (int w = 1; w < (int)(blockDim.x / kWave); ++w) amax = __builtin_fmaxf(amax, wave_max[w]);

    // IEEE float32 division (correctly rounded: the library is compiled without fast-math).
    const float scale = (amax == 0.0f) ? 1.0f : amax / 448.0f;

    for (int i = threadIdx.x; i < row_chunks; i += blockDim.x) {
        const uint4 w = src[i];
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
        uint32_t packed[2] = {0u, 0u};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float2_t f = unpack2(SRC{}, ws[k]);
            const uint32_t c0 = e4m3_encode(f.x / scale);
            const uint32_t c1 = e4m3_encode(f.y / scale);
            packed[k >> 1] |= (c0 | (c1 << 8)) << (16 * (k & 1));
        }
        dst[i] = uint2{packed[0], packed[1]};
    }
    if (threadIdx.x == 0) (is_v ? v_scale : k_scale)[slot] = scale;
}

int threads_for(int64_t items) {
    int64_t n = ((items + kWave - 1) / kWave) * kWave;
    return (int)(n < 256 ? n : 256);
}

}  // namespace

hipError_t launch_append_copy(const void* key, const void* value, void* key_cache, void* value_cache,
                              const int64_t* slots, int64_t num_tokens, int32_t row_bytes,
                              int64_t num_slots, hipStream_t stream) {
    const int32_t row_vec = row_bytes / 16;
    hipLaunchKernelGGL(append_copy_kernel, dim3((uint32_t)num_tokens, 2), dim3(threads_for(row_vec)), 0, stream,
                       (const uint4*)key, (const uint4*)value, (uint4*)key_cache, (uint4*)value_cache, slots,
                       row_vec, num_slots);
    return hipGetLastError();
}

namespace {

hipError_t launch_fp8(const void* key, const void* value, void* key_cache, void* value_cache, float* k_scale,
                      float* v_scale, const SlotSource& src, int64_t num_tokens, int32_t row_elems, int64_t num_slots,
                      int src_kind, hipStream_t stream) {
    const int32_t chunks = row_elems / 8;
    const dim3 grid((uint32_t)num_tokens, 2);
    const dim3 block(threads_for(chunks));
    if (src_kind == kBF16) {
        hipLaunchKernelGGL(append_fp8_kernel<BF16>, grid, block, 0, stream, (const uint4*)key, (const uint4*)value,
                           (uint2*)key_cache, (uint2*)value_cache, k_scale, v_scale, src, chunks, num_slots);
    } else {
        hipLaunchKernelGGL(append_fp8_kernel<F16>, grid, block, 0, stream, (const uint4*)key, (const uint4*)value,
                           (uint2*)key_cache, (uint2*)value_cache, k_scale, v_scale, src, chunks, num_slots);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_append_fp8(const void* key, const void* value, void* key_cache, void* value_cache,
                             float* k_scale, float* v_scale, const int64_t* slots, int64_t num_tokens,
                             int32_t row_elems, int64_t num_slots, int src_kind, hipStream_t stream) {
    return launch_fp8(key, value, key_cache, value_cache, k_scale, v_scale, SlotSource{slots, nullptr, nullptr, 0, 0},
                      num_tokens, row_elems, num_slots, src_kind, stream);
}

hipError_t launch_append_fp8_at_lengths(const void* key, const void* value, void* key_cache, void* value_cache,
                                        float* k_scale, float* v_scale, const int32_t* block_tables,
                                        const int32_t* context_lens, int32_t num_seqs, int32_t max_blocks,
                                        int32_t ctx_limit, int32_t row_elems, int64_t num_slots, int src_kind,
                                        hipStream_t stream) {
    return launch_fp8(key, value, key_cache, value_cache, k_scale, v_scale,
                      SlotSource{nullptr, block_tables, context_lens, max_blocks, ctx_limit}, num_seqs, row_elems,
                      num_slots, src_kind, stream);
}

}  // namespace pa
