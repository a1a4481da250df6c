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
// Work split.  Every wave works alone (no LDS, no barriers) on segments: runs
// of consecutive 16-token blocks of one (sequence, head group), a head group
// being up to 8 query heads that share one KV head.  Two ways to cut the work:
//  * fixed partitions: wave = (sequence, head group, partition of P tokens);
//  * balanced: the (sequence, head group, block) space is laid end to end and
//    cut into equal ranges, one per wave, so long and short sequences cost
//    the same per wave; a range may cover the end of one sequence and the
//    start of the next.
// A segment that covers its whole sequence writes the output row; otherwise
// it writes a partial result (running max m, sum of exponentials l,
// unnormalised V sum) that decode_merge_kernel combines in ascending token
// order, so the output is bitwise deterministic for fixed inputs.
//
// Lane layout.  One 16-byte load per lane; a token's row of one head (D
// elements, 256 bytes for D=128 in 16-bit) is spread over TPL = D*bytes/16
// consecutive lanes, so one wave-wide load covers ROWS = 64/TPL tokens and a
// 16-token block takes LPB = 16/ROWS loads for K and as many for V.  The dot
// product of a row is finished with DPP inside the TPL-lane group.  Each
// group of TPL lanes (a "row") keeps its own online-softmax state over the
// tokens it sees; the rows are merged at the end of a segment.  The loads of
// block j+1 are issued before block j is consumed (two register buffers).
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
    static_assert(TPL == 4 || TPL == 8 || TPL == 16, "row of 4, 8 or 16 lanes");
};

__device__ __forceinline__ int clamp_len(int L, int limit) { return L < 0 ? 0 : (L > limit ? limit : L); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ int seq_len(const DecodeParams& p, int b) { return clamp_len(p.context_lens[b], p.ctx_limit); }

__device__ __forceinline__ int seq_blocks(const DecodeParams& p, int b) {
    return (seq_len(p, b) + kBlockSize - 1) / kBlockSize;
}

// Inclusive prefix sum over the 64 lanes of the wave.
__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    return x;
}

// Blocks of all sequences together (the same value in every lane).
__device__ int total_blocks(const DecodeParams& p, int lane) {
    int total = 0;
    for (int c = 0; c < p.B; c += kWave) {
        const int b = c + lane;
        const int incl = wave_incl_scan(b < p.B ? seq_blocks(p, b) : 0, lane);
        total += __builtin_amdgcn_readlane(incl, kWave - 1);
    }
    return total;
}

struct SeqPos {
    int b;       // sequence
    int start;   // blocks of all earlier sequences
    int nblk;    // blocks of this sequence
};

// The non-empty sequence holding balanced-order position pos, where the
// position of (b, hg, j) is groups * start_b + hg * nblk_b + j and
// 0 <= pos < groups * total_blocks.
__device__ SeqPos locate(const DecodeParams& p, int lane, int pos) {
    int carry = 0;
    for (int c = 0; c < p.B; c += kWave) {
        const int b = c + lane;
        const int nb = b < p.B ? seq_blocks(p, b) : 0;
        const int incl = wave_incl_scan(nb, lane);
        const int start = carry + incl - nb;
        const uint64_t mask = __ballot(nb > 0 && p.groups * start <= pos);
        const int chunk_total = __builtin_amdgcn_readlane(incl, kWave - 1);
        if (p.groups * (carry + chunk_total) > pos) {
            const int lb = 63 - __builtin_clzll(mask);
            return {c + lb, __builtin_amdgcn_readlane(start, lb), __builtin_amdgcn_readlane(nb, lb)};
        }
        carry += chunk_total;
    }
    return {0, 0, 0};
}

// Exclusive block prefix of sequence b.
__device__ int seq_start(const DecodeParams& p, int lane, int b) {
    int carry = 0;
    for (int c = 0; c < p.B; c += kWave) {
        const int bb = c + lane;
        const int nb = bb < p.B ? seq_blocks(p, bb) : 0;
        const int incl = wave_incl_scan(nb, lane);
        if (b < c + kWave) return carry + __builtin_amdgcn_readlane(incl - nb, b - c);
        carry += __builtin_amdgcn_readlane(incl, kWave - 1);
    }
    return carry;
}

// One segment: blocks [jb, je) of sequence b (nblk blocks, L tokens), head group hg.
// Writes the output rows when the segment is the whole sequence, else the partial
// for workspace slot `slot` (HPW consecutive heads per slot).
template <typename QT, typename CT, int D, int HPW>
__device__ __forceinline__ void run_segment(const DecodeParams& p, int lane, int b, int hg, int jb, int je,
                                            int nblk, int L, int64_t slot) {
    using Ly = Layout<CT, D>;
    constexpr int EB = Ly::EB, EPL = Ly::EPL, TPL = Ly::TPL, ROWS = Ly::ROWS, LPB = Ly::LPB;
    constexpr bool kFp8 = EB == 1;

    const int32_t* table = p.block_tables + (int64_t)b * p.max_blocks;
    // Page-table chunk: lane i holds the physical id of logical block jbase + i.
    auto table_chunk = [&](int jbase) {
        const int j = jbase + lane;
        return j < p.max_blocks ? table[j] : -1;
    };
    int tbl = table_chunk(jb);

    const int h0 = hg * HPW;
    const int hk = h0 / (p.Hq / p.Hkv);
    const int row = lane / TPL;
    const int chunk = lane % TPL;

    // Query: this lane's EPL elements of each of the HPW heads.
    uint32_t qw[HPW][4];
    float qf[kFp8 ? HPW : 1][kFp8 ? EPL : 1];
    {
        const uint4* qp = (const uint4*)((const uint16_t*)p.query + ((int64_t)b * p.Hq + h0) * D + chunk * EPL);
#pragma unroll
        for (int h = 0; h < HPW; ++h) {
            if constexpr (!kFp8) {
                const uint4 v = qp[h * D / 8];
                qw[h][0] = v.x; qw[h][1] = v.y; qw[h][2] = v.z; qw[h][3] = v.w;
            } else {
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
    const char* kbase = (const char*)p.key_cache;
    const char* vbase = (const char*)p.value_cache;

    // Issue the loads of logical block j (K, V and, for FP8, the per-token scales), whose
    // physical id is lane j - jbase of `tbl`.  The loads are unconditional so that the
    // compiler can count them exactly (the consumer of the older buffer then waits only for
    // its own loads); an out-of-range physical id reads block 0 instead and the function
    // returns false so that the block is skipped.
    auto issue = [&](int j, int jbase, uint4 (&kr)[LPB], uint4 (&vr)[LPB], float (&ksc)[LPB], float (&vsc)[LPB]) {
        const int phys = __builtin_amdgcn_readlane(tbl, j - jbase);
        const bool ok = phys >= 0 && phys < p.num_blocks;
        const int64_t pb = ok ? phys : 0;
        const char* kb = kbase + pb * blk_bytes;
        const char* vb = vbase + pb * blk_bytes;
#pragma unroll
        for (int i = 0; i < LPB; ++i) kr[i] = *(const uint4*)(kb + lane_off + i * load_step);
#pragma unroll
        for (int i = 0; i < LPB; ++i) vr[i] = *(const uint4*)(vb + lane_off + i * load_step);
        if constexpr (kFp8) {
#pragma unroll
            for (int i = 0; i < LPB; ++i) {
                ksc[i] = p.k_scale[pb * kBlockSize + i * ROWS + row];
                vsc[i] = p.v_scale[pb * kBlockSize + i * ROWS + row];
            }
        }
        return ok;
    };

    // Online-softmax update with the LPB tokens this row holds of block j.
    auto consume = [&](int j, const uint4 (&kr)[LPB], const uint4 (&vr)[LPB], const float (&ksc)[LPB],
                       const float (&vsc)[LPB]) {
        bool valid[LPB];
#pragma unroll
        for (int i = 0; i < LPB; ++i) valid[i] = j * kBlockSize + i * ROWS + row < L;

        float s[LPB][HPW];   // scores in log2 units
#pragma unroll
        for (int i = 0; i < LPB; ++i) {
            if constexpr (!kFp8) {
#pragma unroll
                for (int h = 0; h < HPW; ++h) {
                    float d = 0.0f;
                    d = dot2(CT{}, qw[h][0], kr[i].x, d);
                    d = dot2(CT{}, qw[h][1], kr[i].y, d);
                    d = dot2(CT{}, qw[h][2], kr[i].z, d);
                    d = dot2(CT{}, qw[h][3], kr[i].w, d);
                    d = group_sum<TPL>(d);
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

        // V rows as float32; masked tokens select a zero word.
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
    };

    // Two register buffers: the loads of block j+1 are in flight while block j is consumed.
    // The page table is walked in chunks of 64 blocks (one id per lane).
    uint4 kA[LPB], vA[LPB], kB[LPB], vB[LPB];
    float ksA[LPB], vsA[LPB], ksB[LPB], vsB[LPB];
    for (int jc = jb; jc < je; jc += kWave) {
        if (jc != jb) tbl = table_chunk(jc);
        const int jend = min(je, jc + kWave);
        int j = jc;
        bool okA = issue(j, jc, kA, vA, ksA, vsA);
        while (j + 2 < jend) {
            const bool okB = issue(j + 1, jc, kB, vB, ksB, vsB);
            if (okA) consume(j, kA, vA, ksA, vsA);
            okA = issue(j + 2, jc, kA, vA, ksA, vsA);
            if (okB) consume(j + 1, kB, vB, ksB, vsB);
            j += 2;
        }
        if (j + 1 < jend) {
            const bool okB = issue(j + 1, jc, kB, vB, ksB, vsB);
            if (okA) consume(j, kA, vA, ksA, vsA);
            if (okB) consume(j + 1, kB, vB, ksB, vsB);
        } else if (okA) {
            consume(j, kA, vA, ksA, vsA);
        }
    }

    // Merge the ROWS row states (lanes with equal `chunk`); afterwards every row holds the
    // segment's result and the TPL lanes of row 0 write it.
    const bool whole = jb == 0 && je == nblk;
    const int64_t out_row = (int64_t)b * p.Hq + h0;
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
            if (whole) {
                const float inv = lw > 0.0f ? 1.0f / lw : 0.0f;
                uint32_t packed[EPL / 2];
#pragma unroll
                for (int e = 0; e < EPL / 2; ++e)
                    packed[e] = (uint32_t)to_bits(QT{}, acc[h][2 * e] * inv) |
                                ((uint32_t)to_bits(QT{}, acc[h][2 * e + 1] * inv) << 16);
                uint4* dst = (uint4*)((uint16_t*)p.out + (out_row + h) * D + chunk * EPL);
#pragma unroll
                for (int c = 0; c < EPL / 8; ++c)
                    dst[c] = uint4{packed[4 * c], packed[4 * c + 1], packed[4 * c + 2], packed[4 * c + 3]};
            } else {
                const int64_t hs = slot * HPW + h;
                float4* dst = (float4*)(p.ws_acc + hs * D + chunk * EPL);
#pragma unroll
                for (int c = 0; c < EPL / 4; ++c)
                    dst[c] = float4{acc[h][4 * c], acc[h][4 * c + 1], acc[h][4 * c + 2], acc[h][4 * c + 3]};
                if (chunk == 0) {
                    p.ws_ml[hs * 2] = M;
                    p.ws_ml[hs * 2 + 1] = lw;
                }
            }
        }
    }
}

template <typename QT, typename CT, int D, int HPW>
__global__ __launch_bounds__(kThreads) void decode_kernel(const DecodeParams p) {
    const int lane = threadIdx.x & (kWave - 1);
    const int w = blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    if (w >= p.num_waves) return;

    if (!p.balanced) {
        // Fixed partitions: wave w = (partition, head group, sequence), partition fastest.
        const int part = w % p.NP;
        const int s = w / p.NP;
        const int hg = s % p.groups;
        const int b = s / p.groups;
        const int L = seq_len(p, b);
        const int nblk = (L + kBlockSize - 1) / kBlockSize;
        const int jb = part * p.part_blocks;
        if (jb >= nblk && !(part == 0 && nblk == 0)) return;   // L == 0: partition 0 writes zeros
        const int je = min(nblk, jb + p.part_blocks);
        run_segment<QT, CT, D, HPW>(p, lane, b, hg, jb, je, nblk, L, (int64_t)s * p.NP + part);
        return;
    }

    // Balanced: equal ranges of the (sequence, head group, block) order.
    const int T = p.groups * total_blocks(p, lane);
    const int C = (T + p.num_waves - 1) / p.num_waves;
    int pos = w * C;
    const int pos_end = min(T, pos + C);
    while (pos < pos_end) {
        const SeqPos sp = locate(p, lane, pos);
        const int off = pos - p.groups * sp.start;
        const int hg = off / sp.nblk;
        const int jb = off % sp.nblk;
        const int je = min(sp.nblk, jb + (pos_end - pos));
        const int s = sp.b * p.groups + hg;
        run_segment<QT, CT, D, HPW>(p, lane, sp.b, hg, jb, je, sp.nblk, seq_len(p, sp.b), (int64_t)w + s);
        pos += je - jb;
    }
}

// Merge of the partials of one (sequence, head group): for each head,
// out = sum_k 2^(m_k - M) acc_k / sum_k 2^(m_k - M) l_k over its segments in
// ascending token order.  Also writes the zero rows of empty sequences in the
// balanced split (no segment covers them).
template <typename QT, int D, int HPW>
__global__ __launch_bounds__(kWave * (HPW < 4 ? HPW : 4)) void decode_merge_kernel(const DecodeParams p) {
    constexpr int EPT = D / kWave;
    constexpr int NW = HPW < 4 ? HPW : 4;   // waves, each merging heads wave, wave + NW, ...
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int s = blockIdx.x;
    const int hg = s % p.groups;
    const int b = s / p.groups;
    const int nblk = seq_blocks(p, b);

    int64_t first, count;
    if (!p.balanced) {
        const int n_part = (nblk + p.part_blocks - 1) / p.part_blocks;
        if (n_part <= 1) return;            // written by the one partition (zeros when L == 0)
        first = (int64_t)s * p.NP;
        count = n_part;
    } else {
        const int T = p.groups * total_blocks(p, lane);
        const int C = (T + p.num_waves - 1) / p.num_waves;
        const int pos0 = p.groups * seq_start(p, lane, b) + hg * nblk;
        if (nblk > 0) {
            const int w0 = pos0 / C;
            const int w1 = (pos0 + nblk - 1) / C;
            if (w0 == w1) return;           // one segment: written directly
            first = (int64_t)w0 + s;
            count = w1 - w0 + 1;
        } else {
            first = 0;
            count = 0;
        }
    }

    for (int h = wave; h < HPW; h += NW) {
        const int64_t base = first * HPW + h;   // slot k of this head: (first + k) * HPW + h
        float M = kNegInf;
        for (int k = 0; k < count; ++k) M = __builtin_fmaxf(M, p.ws_ml[(base + (int64_t)k * HPW) * 2]);
        const float ms = (M == kNegInf) ? 0.0f : M;
        float num[EPT];
#pragma unroll
        for (int e = 0; e < EPT; ++e) num[e] = 0.0f;
        float den = 0.0f;
#pragma unroll 4
        for (int k = 0; k < count; ++k) {
            const int64_t hs = base + (int64_t)k * HPW;
            const float f = fast_exp2(p.ws_ml[hs * 2] - ms);
            den = __builtin_fmaf(f, p.ws_ml[hs * 2 + 1], den);
#pragma unroll
            for (int e = 0; e < EPT; ++e) num[e] = __builtin_fmaf(f, p.ws_acc[hs * D + e * kWave + lane], num[e]);
        }
        const int64_t out_row = (int64_t)b * p.Hq + hg * HPW + h;
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            const float o = den > 0.0f ? num[e] / den : 0.0f;
            ((uint16_t*)p.out)[out_row * D + e * kWave + lane] = to_bits(QT{}, o);
        }
    }
}

template <typename QT, typename CT, int D, int HPW>
hipError_t run(const DecodeParams& p, hipStream_t stream) {
    const int64_t grid = ((int64_t)p.num_waves + kWaves - 1) / kWaves;
    hipLaunchKernelGGL((decode_kernel<QT, CT, D, HPW>), dim3((uint32_t)grid), dim3(kThreads), 0, stream, p);
    if (p.balanced || p.NP > 1) {
        hipLaunchKernelGGL((decode_merge_kernel<QT, D, HPW>), dim3((uint32_t)((int64_t)p.B * p.groups)),
                           dim3(kWave * (HPW < 4 ? HPW : 4)), 0, stream, p);
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
