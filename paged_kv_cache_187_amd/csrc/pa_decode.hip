// Paged decode attention for gfx950 (MI355X).
//
// What is computed ("LLM推理引擎深度实战：从PagedAttention到分布式推理部署", §2.2-§2.3): each
// sequence's single new query token attends over all of its cached K/V, which
// live in fixed 16-token physical blocks; the kernel maps logical block j of
// sequence b to its physical block through the page table and reads the rows
// from there, so the result is ordinary softmax attention.  Decode reads
// every cached K/V byte once and does little arithmetic per byte, so the
// kernel is bound by HBM bandwidth ("大模型推理引擎优化：KV Cache 与连续批处理", §一 and
// §4.1): the design goal is to keep enough 16-byte loads in flight, not to
// use the matrix cores.
//
// Work split.  One workgroup (4 waves) per (sequence, group of up to 8 query
// heads sharing one KV head, partition of P tokens).  Sequences longer than
// P are split over several workgroups whose partial results (running max m,
// sum of exponentials l, unnormalised V sum) go to a workspace and are merged
// by decode_reduce_kernel in ascending partition order (deterministic).
//
// Lane layout.  One 16-byte load per lane; a token's row of one head (D
// elements, 256 bytes for D=128 in 16-bit) is spread over TPL = D*bytes/16
// consecutive lanes, so one wave-wide load covers ROWS = 64/TPL tokens and a
// 16-token block takes LPB = 16/ROWS loads for K and as many for V.  The dot
// product of a row is finished with DPP inside the TPL-lane group.  Each
// group of TPL lanes (a "row") keeps its own online-softmax state over the
// tokens it sees; rows and waves are merged once per partition.
//
// Masking.  Tokens at or past the context length are excluded by selection
// (score -> -inf, V word -> 0), never by multiplying, so whatever those
// slots hold (stale data, NaN) cannot reach the output.

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr float kNegInf = -__builtin_huge_valf();

template <typename CT, int D>
struct Layout {
    static constexpr int EB = Storage<CT>::bytes;
    static constexpr int EPL = 16 / EB;            // cache elements per lane per token row
    static constexpr int TPL = D / EPL;            // lanes per token row
    static constexpr int ROWS = kWave / TPL;       // token rows per wave-wide load
    static constexpr int LPB = kBlockSize / ROWS;  // loads per block (K, and again V)
    static constexpr int QW = EPL / 2;             // 32-bit words of 16-bit q per lane (16-bit caches)
    static_assert(TPL == 4 || TPL == 8 || TPL == 16, "row of 4, 8 or 16 lanes");
};

__device__ __forceinline__ int clamp_len(int L, int limit) { return L < 0 ? 0 : (L > limit ? limit : L); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Score of one token row for one head: partial dot product of this lane's
// EPL elements, finished inside the row with DPP.
template <typename QT, typename CT, int D>
struct RowDot;

template <typename T, int D>
struct RowDot16 {
    using L = Layout<T, D>;
    __device__ __forceinline__ static float run(const uint32_t* q, const uint4& k) {
        float d = 0.0f;
        d = dot2(T{}, q[0], k.x, d);
        d = dot2(T{}, q[1], k.y, d);
        d = dot2(T{}, q[2], k.z, d);
        d = dot2(T{}, q[3], k.w, d);
        return group_sum<L::TPL>(d);
    }
};

template <typename QT, typename CT, int D, int HPW>
__global__ __launch_bounds__(kThreads) void decode_partition_kernel(const DecodeParams p) {
    using Ly = Layout<CT, D>;
    constexpr int EB = Ly::EB, EPL = Ly::EPL, TPL = Ly::TPL, ROWS = Ly::ROWS, LPB = Ly::LPB;
    constexpr bool kFp8 = EB == 1;

    __shared__ float sm_m[kWaves][HPW];
    __shared__ float sm_l[kWaves][HPW];
    __shared__ float sm_acc[kWaves][HPW][D];

    // Workgroup -> (partition, head group, sequence); partition index fastest.
    const int wg = blockIdx.x;
    const int part = wg % p.NP;
    const int rest = wg / p.NP;
    const int hg = rest % p.groups;
    const int b = rest / p.groups;

    const int L = clamp_len(p.context_lens[b], p.ctx_limit);
    const int part_tokens = p.part_blocks * kBlockSize;
    const int n_part = L > 0 ? (L + part_tokens - 1) / part_tokens : 1;
    if (part >= n_part) return;

    const int h0 = hg * HPW;
    const int hk = h0 / (p.Hq / p.Hkv);
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int row = lane / TPL;
    const int chunk = lane % TPL;
    const int nblk = (L + kBlockSize - 1) / kBlockSize;
    const int j0 = part * p.part_blocks;
    const int j1 = min(nblk, j0 + p.part_blocks);

    // Query: this lane's EPL elements of each of the HPW heads.
    uint32_t qw[HPW][Ly::QW > 0 ? Ly::QW : 1];
    float qf[kFp8 ? HPW : 1][kFp8 ? EPL : 1];
    {
        const int64_t qbase = ((int64_t)b * p.Hq + h0) * D + chunk * EPL;
        if constexpr (!kFp8) {
            const uint4* qp = (const uint4*)((const uint16_t*)p.query + qbase);
#pragma unroll
            for (int h = 0; h < HPW; ++h) {
                const uint4 v = qp[h * D / 8];
                qw[h][0] = v.x; qw[h][1] = v.y; qw[h][2] = v.z; qw[h][3] = v.w;
            }
        } else {
            const uint4* qp = (const uint4*)((const uint16_t*)p.query + qbase);
#pragma unroll
            for (int h = 0; h < HPW; ++h) {
#pragma unroll
                for (int c = 0; c < EPL / 8; ++c) {
                    const uint4 v = qp[h * D / 8 + c];
                    const uint32_t ws[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const float2_t f = unpack2(QT{}, ws[k]);
                        qf[h][c * 8 + 2 * k] = f.x;
                        qf[h][c * 8 + 2 * k + 1] = f.y;
                    }
                }
            }
        }
    }

    float m[HPW], l[HPW], acc[HPW][EPL];
#pragma unroll
    for (int h = 0; h < HPW; ++h) {
        m[h] = kNegInf;
        l[h] = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = 0.0f;
    }

    const int64_t tok_bytes = (int64_t)p.Hkv * D * EB;         // stride between token rows
    const int64_t blk_bytes = tok_bytes * kBlockSize;
    const uint32_t lane_off = (uint32_t)(row * tok_bytes + (int64_t)hk * D * EB + chunk * 16);
    const uint32_t load_step = (uint32_t)(ROWS * tok_bytes);
    const int32_t* table = p.block_tables + (int64_t)b * p.max_blocks;
    const char* kbase = (const char*)p.key_cache;
    const char* vbase = (const char*)p.value_cache;

    for (int j = j0 + wave; j < j1; j += kWaves) {
        const int phys = table[j];
        if (phys < 0 || phys >= p.num_blocks) continue;   // invalid id: block skipped
        const char* kb = kbase + (int64_t)phys * blk_bytes;
        const char* vb = vbase + (int64_t)phys * blk_bytes;
        uint4 kr[LPB], vr[LPB];
#pragma unroll
        for (int i = 0; i < LPB; ++i) kr[i] = *(const uint4*)(kb + lane_off + i * load_step);
#pragma unroll
        for (int i = 0; i < LPB; ++i) vr[i] = *(const uint4*)(vb + lane_off + i * load_step);
        float ksc[LPB], vsc[LPB];
        if constexpr (kFp8) {
#pragma unroll
            for (int i = 0; i < LPB; ++i) {
                ksc[i] = p.k_scale[(int64_t)phys * kBlockSize + i * ROWS + row];
                vsc[i] = p.v_scale[(int64_t)phys * kBlockSize + i * ROWS + row];
            }
        }

        bool valid[LPB];
#pragma unroll
        for (int i = 0; i < LPB; ++i) valid[i] = j * kBlockSize + i * ROWS + row < L;

        // Scores (already in log2 units).
        float s[LPB][HPW];
#pragma unroll
        for (int i = 0; i < LPB; ++i) {
            if constexpr (!kFp8) {
#pragma unroll
                for (int h = 0; h < HPW; ++h) {
                    const float d = RowDot16<CT, D>::run(qw[h], kr[i]);
                    s[i][h] = valid[i] ? d * p.scale_log2 : kNegInf;
                }
            } else {
                float kf[EPL];
                unpack4_fp8(kr[i].x, kf + 0);
                unpack4_fp8(kr[i].y, kf + 4);
                unpack4_fp8(kr[i].z, kf + 8);
                unpack4_fp8(kr[i].w, kf + 12);
                const float sc = p.scale_log2 * ksc[i];
#pragma unroll
                for (int h = 0; h < HPW; ++h) {
                    float d = 0.0f;
#pragma unroll
                    for (int e = 0; e < EPL; ++e) d = __builtin_fmaf(qf[h][e], kf[e], d);
                    d = group_sum<TPL>(d);
                    s[i][h] = valid[i] ? d * sc : kNegInf;
                }
            }
        }

        // V rows as float32, zero for masked tokens.
        float vf[LPB][EPL];
#pragma unroll
        for (int i = 0; i < LPB; ++i) {
            const uint32_t w[4] = {valid[i] ? vr[i].x : 0u, valid[i] ? vr[i].y : 0u, valid[i] ? vr[i].z : 0u,
                                   valid[i] ? vr[i].w : 0u};
            if constexpr (!kFp8) {
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const float2_t f = unpack2(CT{}, w[k]);
                    vf[i][2 * k] = f.x;
                    vf[i][2 * k + 1] = f.y;
                }
            } else {
#pragma unroll
                for (int k = 0; k < 4; ++k) unpack4_fp8(w[k], &vf[i][4 * k]);
            }
        }

        // Online softmax update of each head over this block's LPB tokens of this row.
#pragma unroll
        for (int h = 0; h < HPW; ++h) {
            float mb = s[0][h];
#pragma unroll
            for (int i = 1; i < LPB; ++i) mb = __builtin_fmaxf(mb, s[i][h]);
            const float mn = __builtin_fmaxf(m[h], mb);
            const float ms = (mn == kNegInf) ? 0.0f : mn;
            const float alpha = fast_exp2(m[h] - ms);
            float pr[LPB];
            float psum = 0.0f;
#pragma unroll
            for (int i = 0; i < LPB; ++i) {
                pr[i] = fast_exp2(s[i][h] - ms);
                psum += pr[i];
                if constexpr (kFp8) pr[i] = valid[i] ? pr[i] * vsc[i] : 0.0f;
            }
            l[h] = l[h] * alpha + psum;
            m[h] = mn;
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                float a = acc[h][e] * alpha;
#pragma unroll
                for (int i = 0; i < LPB; ++i) a = __builtin_fmaf(pr[i], vf[i][e], a);
                acc[h][e] = a;
            }
        }
    }

    // Merge the ROWS row states of this wave (lanes with equal `chunk`).
#pragma unroll
    for (int h = 0; h < HPW; ++h) {
        float M = m[h];
#pragma unroll
        for (int off = TPL; off < kWave; off <<= 1) M = __builtin_fmaxf(M, __shfl_xor(M, off));
        const float w = fast_exp2(m[h] - ((M == kNegInf) ? 0.0f : M));
        float lw = l[h] * w;
#pragma unroll
        for (int off = TPL; off < kWave; off <<= 1) lw += __shfl_xor(lw, off);
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            float a = acc[h][e] * w;
#pragma unroll
            for (int off = TPL; off < kWave; off <<= 1) a += __shfl_xor(a, off);
            acc[h][e] = a;
        }
        if (row == 0) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) sm_acc[wave][h][chunk * EPL + e] = acc[h][e];
            if (chunk == 0) {
                sm_m[wave][h] = M;
                sm_l[wave][h] = lw;
            }
        }
    }
    __syncthreads();

    // Merge the waves; write the output row (one partition) or the partial.
    for (int idx = threadIdx.x; idx < HPW * D; idx += kThreads) {
        const int h = idx / D;
        const int d = idx % D;
        float M = sm_m[0][h];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) M = __builtin_fmaxf(M, sm_m[w][h]);
        const float ms = (M == kNegInf) ? 0.0f : M;
        float num = 0.0f, den = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float f = fast_exp2(sm_m[w][h] - ms);
            num = __builtin_fmaf(f, sm_acc[w][h][d], num);
            den = __builtin_fmaf(f, sm_l[w][h], den);
        }
        const int head = h0 + h;
        if (n_part == 1) {
            const float o = den > 0.0f ? num / den : 0.0f;
            ((uint16_t*)p.out)[((int64_t)b * p.Hq + head) * D + d] = to_bits(QT{}, o);
        } else {
            const int64_t slot = ((int64_t)b * p.Hq + head) * p.NP + part;
            p.ws_acc[slot * D + d] = num;
            if (d == 0) {
                p.ws_ml[slot * 2] = M;
                p.ws_ml[slot * 2 + 1] = den;
            }
        }
    }
}

// Merge of the partition partials of one (sequence, head), ascending partition
// order: out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p.
template <typename QT, int D>
__global__ __launch_bounds__(kWave) void decode_reduce_kernel(const DecodeParams p) {
    constexpr int EPT = D / kWave;
    const int h = blockIdx.x % p.Hq;
    const int b = blockIdx.x / p.Hq;
    const int L = clamp_len(p.context_lens[b], p.ctx_limit);
    const int part_tokens = p.part_blocks * kBlockSize;
    const int n_part = L > 0 ? (L + part_tokens - 1) / part_tokens : 1;
    if (n_part <= 1) return;   // written directly by the partition kernel

    const int64_t base = ((int64_t)b * p.Hq + h) * p.NP;
    const float* ml = p.ws_ml + base * 2;
    const float* accp = p.ws_acc + base * D;
    float M = kNegInf;
    for (int q = 0; q < n_part; ++q) M = __builtin_fmaxf(M, ml[2 * q]);
    const float ms = (M == kNegInf) ? 0.0f : M;
    float num[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) num[e] = 0.0f;
    float den = 0.0f;
    const int lane = threadIdx.x;
#pragma unroll 4
    for (int q = 0; q < n_part; ++q) {
        const float f = fast_exp2(ml[2 * q] - ms);
        den = __builtin_fmaf(f, ml[2 * q + 1], den);
#pragma unroll
        for (int e = 0; e < EPT; ++e) num[e] = __builtin_fmaf(f, accp[(int64_t)q * D + e * kWave + lane], num[e]);
    }
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        const float o = den > 0.0f ? num[e] / den : 0.0f;
        ((uint16_t*)p.out)[((int64_t)b * p.Hq + h) * D + e * kWave + lane] = to_bits(QT{}, o);
    }
}

template <typename QT, typename CT, int D, int HPW>
hipError_t run(const DecodeParams& p, hipStream_t stream) {
    const int64_t grid = (int64_t)p.NP * p.groups * p.B;
    hipLaunchKernelGGL((decode_partition_kernel<QT, CT, D, HPW>), dim3((uint32_t)grid), dim3(kThreads), 0, stream,
                       p);
    if (p.NP > 1) {
        hipLaunchKernelGGL((decode_reduce_kernel<QT, D>), dim3((uint32_t)((int64_t)p.B * p.Hq)), dim3(kWave), 0,
                           stream, p);
    }
    return hipGetLastError();
}

template <typename QT, typename CT, int D>
hipError_t run_hpw(const DecodeParams& p, int hpw, hipStream_t s) {
    switch (hpw) {
        case 1: return run<QT, CT, D, 1>(p, s);
        case 2: return run<QT, CT, D, 2>(p, s);
        case 4: return run<QT, CT, D, 4>(p, s);
        case 8: return run<QT, CT, D, 8>(p, s);
        default: return hipErrorInvalidValue;
    }
}

template <typename QT, typename CT>
hipError_t run_d(const DecodeParams& p, int d, int hpw, hipStream_t s) {
    switch (d) {
        case 64: return run_hpw<QT, CT, 64>(p, hpw, s);
        case 128: return run_hpw<QT, CT, 128>(p, hpw, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

int heads_per_workgroup(int group) {
    for (int h = 8; h > 1; h >>= 1)
        if (group % h == 0) return h;
    return 1;
}

hipError_t launch_decode(const DecodeParams& p, int head_dim, int q_kind, int cache_kind, int hpw,
                         hipStream_t stream) {
    if (q_kind == kF16 && cache_kind == kF16) return run_d<F16, F16>(p, head_dim, hpw, stream);
    if (q_kind == kBF16 && cache_kind == kBF16) return run_d<BF16, BF16>(p, head_dim, hpw, stream);
    if (q_kind == kF16 && cache_kind == kFP8) return run_d<F16, FP8>(p, head_dim, hpw, stream);
    if (q_kind == kBF16 && cache_kind == kFP8) return run_d<BF16, FP8>(p, head_dim, hpw, stream);
    return hipErrorInvalidValue;
}

}  // namespace pa
