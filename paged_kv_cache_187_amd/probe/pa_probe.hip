// Read-bandwidth probes for gfx950, used only to report the achievable ceiling next
// to the decode measurements (built as libpaprobe.so, not part of libpagedattn.so).
//
//  * pa_probe_stream: a plain streaming read of a contiguous buffer.
//  * pa_probe_gather: the paged-decode access pattern without the attention: for every
//    (head, position) pair, the 16 rows of one head of a block reached through an id
//    list (128- or 256-byte rows: 128 one-byte or 16-bit values; a token row of all heads
//    apart), in head-major order cut into equal ranges, one per wave, with the next
//    block's loads issued before the current one is used.
//  * pa_probe_gather_teams: the same rows in the decode's order: waves come in teams of
//    one per head, and the waves of a team read the same range of blocks, each its own
//    head's rows.
// Both XOR the loaded words into one word per lane of `sink` so the loads are kept.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kWave = 64;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
// Keeps the compiler from moving memory operations (and the scheduler from moving any
// instruction) across this point.
__device__ __forceinline__ void order_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
}
__device__ __forceinline__ uint4 load_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 2));
}

__global__ __launch_bounds__(256) void stream_kernel(const uint4* __restrict__ buf, int64_t n_vec,
                                                     uint32_t* __restrict__ sink) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    uint32_t acc = 0;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_vec; i += stride) {
        const u32x4_t v = __builtin_nontemporal_load((const u32x4_t*)buf + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

// One wave per range of (head, position) pairs.  ROW-byte rows: ROW / 16 lanes per row,
// 1024 / ROW rows per 16-byte-per-lane load, ROW / 64 loads per 16-row block.
template <int ROW>
__global__ __launch_bounds__(256) void gather_kernel(const char* __restrict__ pool, const int32_t* __restrict__ ids,
                                                     int32_t n_ids, int32_t hkv, int64_t num_blocks,
                                                     int32_t waves, uint32_t* __restrict__ sink) {
    constexpr int LPR = ROW / 16;                      // lanes per row
    constexpr int RPL = kWave / LPR;                   // rows per load
    constexpr int NL = 16 / RPL;                       // loads per block
    const int lane = threadIdx.x & (kWave - 1);
    const int w = blockIdx.x * (blockDim.x / kWave) + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    if (w >= waves) return;
    const int64_t tok = (int64_t)hkv * ROW;            // bytes between token rows
    const int64_t blk = tok * 16;
    const int64_t T = (int64_t)hkv * n_ids;
    const int64_t C = (T + waves - 1) / waves;
    const int64_t lo = (int64_t)w * C < T ? (int64_t)w * C : T;
    const int64_t hi = lo + C < T ? lo + C : T;
    const uint32_t lane_off = (uint32_t)((lane / LPR) * tok + (lane % LPR) * 16);
    uint32_t acc = 0;
    auto issue = [&](int64_t q, uint4* b) {
        const bool ok = q < hi;
        int64_t id = 0;
        int head = 0;
        if (ok) {
            head = (int)(q / n_ids);
            id = ids[q % n_ids];
            if (id < 0 || id >= num_blocks) id = 0;
        }
        const auto r = rsrc(pool + id * blk, ok ? (int)blk : 0);
        const uint32_t off = lane_off + (uint32_t)head * ROW;
#pragma unroll
        for (int i = 0; i < NL; ++i) b[i] = load_nt(r, off + (uint32_t)(i * RPL * tok));
    };
    uint4 a[NL], b[NL];
    issue(lo, a);
    for (int64_t q = lo; q < hi; q += 2) {
        issue(q + 1, b);
        order_barrier();
#pragma unroll
        for (int i = 0; i < NL; ++i) acc ^= a[i].x ^ a[i].y ^ a[i].z ^ a[i].w;
        issue(q + 2, a);
        order_barrier();
        if (q + 1 < hi) {
#pragma unroll
            for (int i = 0; i < NL; ++i) acc ^= b[i].x ^ b[i].y ^ b[i].z ^ b[i].w;
        }
    }
    sink[(int64_t)w * kWave + lane] = acc;
}

// Teams of hkv waves: wave w reads head w % hkv of the blocks in range w / hkv, the
// ranges cutting the id list into waves / hkv pieces whose lengths differ by at most one.
template <int ROW>
__global__ __launch_bounds__(256) void gather_teams_kernel(const char* __restrict__ pool,
                                                           const int32_t* __restrict__ ids, int32_t n_ids,
                                                           int32_t hkv, int64_t num_blocks, int32_t waves,
                                                           uint32_t* __restrict__ sink) {
    constexpr int LPR = ROW / 16;
    constexpr int RPL = kWave / LPR;
    constexpr int NL = 16 / RPL;
    const int lane = threadIdx.x & (kWave - 1);
    const int w = blockIdx.x * (blockDim.x / kWave) + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    if (w >= waves) return;
    const int64_t tok = (int64_t)hkv * ROW;
    const int64_t blk = tok * 16;
    const int head = w % hkv;
    const int64_t teams = waves / hkv, r = w / hkv;
    const int64_t lo = r * n_ids / teams, hi = (r + 1) * n_ids / teams;
    const uint32_t off0 = (uint32_t)((lane / LPR) * tok + (lane % LPR) * 16 + (int64_t)head * ROW);
    uint32_t acc = 0;
    auto issue = [&](int64_t q, uint4* b) {
        const bool ok = q < hi;
        int64_t id = 0;
        if (ok) {
            id = ids[q];
            if (id < 0 || id >= num_blocks) id = 0;
        }
        const auto rs = rsrc(pool + id * blk, ok ? (int)blk : 0);
#pragma unroll
        for (int i = 0; i < NL; ++i) b[i] = load_nt(rs, off0 + (uint32_t)(i * RPL * tok));
    };
    // The next block's loads must go out before the current block is used: without the
    // barriers the compiler sinks them below the use and keeps one block in flight.
    uint4 a[NL], b[NL];
    issue(lo, a);
    for (int64_t q = lo; q < hi; q += 2) {
        issue(q + 1, b);
        order_barrier();
#pragma unroll
        for (int i = 0; i < NL; ++i) acc ^= a[i].x ^ a[i].y ^ a[i].z ^ a[i].w;
        issue(q + 2, a);
        order_barrier();
        if (q + 1 < hi) {
#pragma unroll
            for (int i = 0; i < NL; ++i) acc ^= b[i].x ^ b[i].y ^ b[i].z ^ b[i].w;
        }
    }
    sink[(int64_t)w * kWave + lane] = acc;
}

}  // namespace

extern "C" {

// Streaming read of `bytes` (a multiple of 16) from `buf`; sink holds one word per
// thread of the grid (blocks * 256 words).  Returns a hipError_t value.
int pa_probe_stream(const void* buf, int64_t bytes, uint32_t* sink, int32_t blocks, void* stream) {
    if (!buf || !sink || bytes <= 0 || bytes % 16 || blocks <= 0) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(stream_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (const uint4*)buf,
                       bytes / 16, sink);
    return (int)hipGetLastError();
}

// Paged gather over a pool of `num_blocks` blocks [16, hkv, row_bytes] (row_bytes 128 or
// 256): every head of every listed block, `waves` waves; sink holds waves * 64 words.
// Ids outside [0, num_blocks) read block 0.  Returns a hipError_t value.
int pa_probe_gather(const void* pool, const int32_t* ids, int32_t n_ids, int32_t hkv, int32_t row_bytes,
                    int64_t num_blocks, int32_t waves, uint32_t* sink, void* stream) {
    if (!pool || !ids || !sink || n_ids <= 0 || hkv <= 0 || num_blocks <= 0 || waves <= 0 ||
        (row_bytes != 128 && row_bytes != 256) || (int64_t)hkv * row_bytes * 16 > (int64_t)1 << 30)
        return (int)hipErrorInvalidValue;
    const dim3 grid((waves + 3) / 4);
    if (row_bytes == 128)
        hipLaunchKernelGGL(gather_kernel<128>, grid, dim3(256), 0, (hipStream_t)stream, (const char*)pool, ids,
                           n_ids, hkv, num_blocks, waves, sink);
    else
        hipLaunchKernelGGL(gather_kernel<256>, grid, dim3(256), 0, (hipStream_t)stream, (const char*)pool, ids,
                           n_ids, hkv, num_blocks, waves, sink);
    return (int)hipGetLastError();
}

// The gather in the decode's team order (waves a multiple of hkv); arguments and sink as
// pa_probe_gather.  Returns a hipError_t value.
int pa_probe_gather_teams(const void* pool, const int32_t* ids, int32_t n_ids, int32_t hkv, int32_t row_bytes,
                          int64_t num_blocks, int32_t waves, uint32_t* sink, void* stream) {
    if (!pool || !ids || !sink || n_ids <= 0 || hkv <= 0 || num_blocks <= 0 || waves <= 0 || waves % hkv != 0 ||
        (row_bytes != 128 && row_bytes != 256) || (int64_t)hkv * row_bytes * 16 > (int64_t)1 << 30)
        return (int)hipErrorInvalidValue;
    const dim3 grid((waves + 3) / 4);
    if (row_bytes == 128)
        hipLaunchKernelGGL(gather_teams_kernel<128>, grid, dim3(256), 0, (hipStream_t)stream, (const char*)pool, ids,
                           n_ids, hkv, num_blocks, waves, sink);
    else
        hipLaunchKernelGGL(gather_teams_kernel<256>, grid, dim3(256), 0, (hipStream_t)stream, (const char*)pool, ids,
                           n_ids, hkv, num_blocks, waves, sink);
    return (int)hipGetLastError();
}

}  // extern "C"
