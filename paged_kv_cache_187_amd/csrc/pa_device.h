// Device-side helpers shared by the gfx950 kernels: storage-type traits,
// 16-lane DPP row reductions, and the FP8 E4M3 encoder used by the
// quantising append.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kBlockSize = 16;   // tokens per physical KV block (fixed)
constexpr int kWave = 64;        // CDNA wavefront width

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));

// Storage kinds of the KV cache and of Q / out.
struct F16 {};
struct BF16 {};
struct FP8 {};

template <typename T> struct Storage;
template <> struct Storage<F16> { static constexpr int bytes = 2; };
template <> struct Storage<BF16> { static constexpr int bytes = 2; };
template <> struct Storage<FP8> { static constexpr int bytes = 1; };

// ---------------------------------------------------------------------------
// Streaming loads.  K/V bytes are read once per decode, so their loads carry the
// non-temporal hint: they do not displace the page tables, queries and partial
// results that other waves reuse from the caches (measured: +16 % read bandwidth for
// the decode's access pattern on gfx950).

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 load_stream(const uint4* p) {
    return __builtin_bit_cast(uint4, __builtin_nontemporal_load((const u32x4_t*)p));
}
__device__ __forceinline__ uint2 load_stream(const uint2* p) {
    return __builtin_bit_cast(uint2, __builtin_nontemporal_load((const u32x2_t*)p));
}
__device__ __forceinline__ uint32_t load_stream(const uint32_t* p) { return __builtin_nontemporal_load(p); }
// Loads through a buffer descriptor that covers `bytes` bytes from `base`: lanes whose
// offset falls outside the range read zeros without touching memory (a descriptor of 0
// bytes turns a load into a no-op that still counts as an issued load).  kStream marks
// the loads non-temporal.
constexpr int kBufferConfig = 0x00020000;   // raw (untyped) buffer access on gfx9
constexpr int kCacheNormal = 0;
constexpr int kCacheStream = 2;             // nt: read once, evict first

__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kBufferConfig);
}
template <int POLICY>
__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, POLICY));
}
template <int POLICY>
__device__ __forceinline__ uint2 buffer_load8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, POLICY));
}
template <int POLICY>
__device__ __forceinline__ uint32_t buffer_load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, POLICY);
}

__device__ __forceinline__ void store_stream(uint4* p, uint4 v) {
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, v), (u32x4_t*)p);
}

// ---------------------------------------------------------------------------
// Conversions of packed 32-bit words to float32 (all exact).

// Two 16-bit floats packed in one word -> two float32 (element 0 = low half).
__device__ __forceinline__ float2_t unpack2(F16, uint32_t w) {
    half2_t h = __builtin_bit_cast(half2_t, w);
    return float2_t{(float)h.x, (float)h.y};
}
__device__ __forceinline__ float2_t unpack2(BF16, uint32_t w) {
    return float2_t{__uint_as_float(w << 16), __uint_as_float(w & 0xFFFF0000u)};
}
// Four E4M3 codes in one word -> four float32, via the gfx950 converter
// (bytes 0,1 then 2,3).
__device__ __forceinline__ void unpack4_fp8(uint32_t w, float* f) {
    float2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
    float2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
    f[0] = lo.x; f[1] = lo.y; f[2] = hi.x; f[3] = hi.y;
}

// float32 -> storage, round to nearest even.
__device__ __forceinline__ uint16_t to_bits(F16, float x) {
    return __builtin_bit_cast(uint16_t, (_Float16)x);
}
__device__ __forceinline__ uint16_t to_bits(BF16, float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// Dot product of two words holding 2 packed 16-bit floats each, accumulated
// into float32 (v_dot2c_f32_f16 / v_dot2c_f32_bf16).
__device__ __forceinline__ float dot2(F16, uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c, false);
}
__device__ __forceinline__ float dot2(BF16, uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, a), __builtin_bit_cast(bf162_t, b), c,
                                           false);
}

// ---------------------------------------------------------------------------
// Lane-group reductions.  DPP row operations act inside rows of 16 lanes:
// quad_perm swaps inside quads, row_half_mirror maps lane i to 7-i inside
// each 8-lane half row, row_mirror maps i to 15-i inside the row.  After the
// quad steps all lanes of a quad hold the same value, so a mirror pairs every
// lane with one of the other quad (or half row) and the sum is complete.

constexpr int kDppQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kDppRowMirror = 0x140;
constexpr int kDppRowHalfMirror = 0x141;

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Sum over aligned groups of N lanes (N = 4, 8 or 16); every lane of the group
// gets the group's sum.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(N == 4 || N == 8 || N == 16, "group of 4, 8 or 16 lanes");
    x += dpp<kDppQuadXor1>(x);
    x += dpp<kDppQuadXor2>(x);
    if constexpr (N >= 8) x += dpp<kDppRowHalfMirror>(x);
    if constexpr (N >= 16) x += dpp<kDppRowMirror>(x);
    return x;
}

// ---------------------------------------------------------------------------
// float32 -> OCP E4M3 (fn) code: round to nearest, ties to even, magnitudes
// of 448 and above (and Inf) saturate to 448; NaN -> 0x7F; the sign bit is
// kept (so -0.0 -> 0x80).  Integer-exact: below 2^-6 the code is the integer
// nearest to |y| * 2^9; above, the top three fraction bits of |y| with a
// round-half-even carry that may step into the next exponent.
__device__ __forceinline__ uint32_t e4m3_encode(float y) {
    const uint32_t u = __float_as_uint(y);
    const uint32_t sign = (u >> 24) & 0x80u;
    const float a = __builtin_fabsf(y);
    uint32_t mag;
    if (!(a < 448.0f)) {
        mag = (a != a) ? 0x7Fu : 0x7Eu;
    } else if (a < 0.015625f) {
        mag = (uint32_t)__builtin_rintf(a * 512.0f);
    } else {
        const uint32_t ua = __float_as_uint(a);
        const uint32_t frac = ua & 0x7FFFFFu;
        mag = (((ua >> 23) - 120u) << 3) | (frac >> 20);
        const uint32_t rest = frac & 0xFFFFFu;
        if (rest > 0x80000u || (rest == 0x80000u && (mag & 1u))) mag += 1u;
    }
    return sign | mag;
}

// ---------------------------------------------------------------------------
// 16x16 matrix-core tiles (fp32 accumulate) in operand type M (F16 or BF16).
// Lane layouts (wave64, checked on gfx950): for the 16x16x32 shape lane l holds
// A[l%16][8*(l/16)+i] and B[8*(l/16)+i][l%16], i < 8; for 16x16x16 the same with
// 4*(l/16)+i, i < 4; the fp32 result holds C[4*(l/16)+r][l%16], r < 4.

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <typename M>
struct Mma;

template <>
struct Mma<BF16> {
    static __device__ __forceinline__ f32x4_t k32(uint4 a, uint4 b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                      c, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4_t k16(uint2 a, uint2 b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a),
                                                         __builtin_bit_cast(s16x4_t, b), c, 0, 0, 0);
    }
    // Two floats -> one packed pair, rounded toward zero (exact for values the type holds).
    static __device__ __forceinline__ uint32_t pack_rtz(float lo, float hi) {
        return (__float_as_uint(hi) & 0xFFFF0000u) | (__float_as_uint(lo) >> 16);
    }
    // E4M3 codes in bytes 2*SEL, 2*SEL+1 of w -> one packed pair (exact: every E4M3 value
    // is a bf16 value; the scale is 1).
    template <bool SEL>
    static __device__ __forceinline__ uint32_t widen2(uint32_t w) {
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, SEL));
    }
};

template <>
struct Mma<F16> {
    static __device__ __forceinline__ f32x4_t k32(uint4 a, uint4 b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                     0, 0, 0);
    }
    static __device__ __forceinline__ f32x4_t k16(uint2 a, uint2 b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a), __builtin_bit_cast(f16x4_t, b), c,
                                                    0, 0, 0);
    }
    static __device__ __forceinline__ uint32_t pack_rtz(float lo, float hi) {
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
    }
    // E4M3 codes in bytes 2*SEL, 2*SEL+1 of w -> one packed pair (exact: every E4M3 value
    // is an f16 value; the scale is 1).
    template <bool SEL>
    static __device__ __forceinline__ uint32_t widen2(uint32_t w) {
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, SEL));
    }
};

}  // namespace pa
