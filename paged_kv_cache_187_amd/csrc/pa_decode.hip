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
// Work split.  Every wave works alone (no barriers; the matrix-core path uses a
// per-wave LDS tile) on segments: runs of consecutive 16-token blocks of one
// (sequence, head group), a head group being the query heads of one KV head
// that one wave serves.  The waves come in teams of one wave per head group:
// the waves of a team read the same blocks at about the same time, each its
// own head's rows, so every block is fetched whole (all heads) within a short
// window, which the memory system serves faster than the same rows spread
// over the kernel's whole run.  Two ways to cut the work:
//  * fixed partitions: team = (sequence, partition of P tokens);
//  * balanced: the (sequence, block) positions are laid end to end and cut
//    into equal ranges, one per team, so long and short sequences cost the
//    same per wave; a range may cover the end of one sequence and the start
//    of the next.
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

// First token a query attends to: with a sliding window of W tokens only the last
// W of the L tokens count ("LLM推理引擎深度实战：…", §9.2 names sliding-window attention).
__device__ __forceinline__ int first_token(const DecodeParams& p, int L) {
    return (p.window > 0 && L > p.window) ? L - p.window : 0;
}

// Blocks of sequence b that hold tokens the query attends to ("in play"): from the
// block of its first attended token to its last block.
__device__ __forceinline__ int seq_blocks(const DecodeParams& p, int b) {
    const int L = seq_len(p, b);
    return L > 0 ? (L + kBlockSize - 1) / kBlockSize - first_token(p, L) / kBlockSize : 0;
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

// Shared-prefix groups.  The prefix of group gi is its first prefix_blocks[gi] blocks,
// clamped to the shortest sequence of the group (every sequence holds all of them).
// Blocks a unit of group gi reads: the shared prefix once, then every sequence's blocks
// after it.  (At most 16 sequences per group: the loads are issued together.)
__device__ int group_blocks(const DecodeParams& p, int gi) {
    int nb[16];
#pragma unroll
    for (int s = 0; s < 16; ++s) nb[s] = s < p.sgroup ? seq_blocks(p, gi * p.sgroup + s) : 0;
    const int P0 = p.prefix_blocks[gi];
    int sum = 0, mn = 0x7fffffff;
#pragma unroll
    for (int s = 0; s < 16; ++s) {
        sum += nb[s];
        if (s < p.sgroup) mn = min(mn, nb[s]);
    }
    const int P = P0 < 0 ? 0 : (P0 > mn ? mn : P0);
    return sum - (p.sgroup - 1) * P;
}

// Entries of the balanced order: sequences, or shared-prefix groups of sequences.
__device__ __forceinline__ int num_entries(const DecodeParams& p) { return p.sgroup > 0 ? p.B / p.sgroup : p.B; }
__device__ __forceinline__ int entry_blocks(const DecodeParams& p, int e) {
    return p.sgroup > 0 ? group_blocks(p, e) : seq_blocks(p, e);
}

// Blocks of all entries together (the same value in every lane).
__device__ int total_blocks(const DecodeParams& p, int lane) {
    const int n = num_entries(p);
    int total = 0;
    for (int c = 0; c < n; c += kWave) {
        const int b = c + lane;
        const int incl = wave_incl_scan(b < n ? entry_blocks(p, b) : 0, lane);
        total += __builtin_amdgcn_readlane(incl, kWave - 1);
    }
    return total;
}

struct SeqPos {
    int b;       // entry: sequence, or shared-prefix group
    int start;   // blocks of all earlier entries
    int nblk;    // blocks of this entry
};

// Block counts of the entries, read once per wave: lane b holds entry b's block count
// and exclusive block prefix when there are at most 64 entries (`single`); otherwise
// the lookups below walk the lengths 64 at a time.
struct SeqTable {
    int nb, start, total;
    bool single;
};

__device__ SeqTable seq_table(const DecodeParams& p, int lane) {
    SeqTable st;
    const int n = num_entries(p);
    st.single = n <= kWave;
    st.nb = lane < n ? entry_blocks(p, lane) : 0;
    const int incl = wave_incl_scan(st.nb, lane);
    st.start = incl - st.nb;
    st.total = st.single ? __builtin_amdgcn_readlane(incl, kWave - 1) : total_blocks(p, lane);
    return st;
}

// A wave's walk through the balanced order.  The lanes hold 64 consecutive entries
// c .. c + 63: entry c + lane's clamped length (sequences; 0 for groups, whose segments
// read their own lengths), block count and first position.  Positions only grow along a
// wave's range, so the walk loads each chunk once and a new segment's entry is a ballot
// over registers, with no memory access.
struct Cursor {
    int c, len, nb, start, end;   // end: the position after the chunk's last entry
};

__device__ Cursor cursor_chunk(const DecodeParams& p, int lane, int c, int carry) {
    Cursor k;
    const int n = num_entries(p);
    const int b = c + lane;
    k.c = c;
    if (p.sgroup > 0) {
        k.len = 0;
        k.nb = b < n ? group_blocks(p, b) : 0;
    } else {
        k.len = b < n ? seq_len(p, b) : 0;
        k.nb = k.len > 0 ? (k.len + kBlockSize - 1) / kBlockSize - first_token(p, k.len) / kBlockSize : 0;
    }
    const int incl = wave_incl_scan(k.nb, lane);
    k.start = carry + incl - k.nb;
    k.end = carry + __builtin_amdgcn_readlane(incl, kWave - 1);
    return k;
}

// The non-empty entry holding position pos (0 <= pos < total blocks), moving the cursor on.
__device__ SeqPos cursor_find(const DecodeParams& p, int lane, Cursor& k, int pos, int& len) {
    while (pos >= k.end) k = cursor_chunk(p, lane, k.c + kWave, k.end);
    const uint64_t mask = __ballot(k.nb > 0 && k.start <= pos);
    const int lb = 63 - __builtin_clzll(mask);
    len = __builtin_amdgcn_readlane(k.len, lb);
    return {k.c + lb, __builtin_amdgcn_readlane(k.start, lb), __builtin_amdgcn_readlane(k.nb, lb)};
}

// Block count and exclusive block prefix of entry b (b wave-uniform).
__device__ SeqPos seq_entry(const DecodeParams& p, const SeqTable& st, int lane, int b) {
    if (st.single) return {b, __builtin_amdgcn_readlane(st.start, b), __builtin_amdgcn_readlane(st.nb, b)};
    const int n = num_entries(p);
    int carry = 0;
    for (int c = 0; c < n; c += kWave) {
        const int bb = c + lane;
        const int nb = bb < n ? entry_blocks(p, bb) : 0;
        const int incl = wave_incl_scan(nb, lane);
        if (b < c + kWave)
            return {b, carry + __builtin_amdgcn_readlane(incl - nb, b - c), __builtin_amdgcn_readlane(nb, b - c)};
        carry += __builtin_amdgcn_readlane(incl, kWave - 1);
    }
    return {b, carry, 0};
}

// Ranges of the balanced split: the T block positions are cut into n <= teams ranges
// whose lengths differ by at most one (range r is [floor(r T / n), floor((r + 1) T / n))),
// each running on one team of `groups` waves, one per head group (team r when there are as
// many ranges as teams).  Range boundaries depend only on the lengths and the launch shape.  The partial
// of entry e, head group hg from range r goes to workspace slot hg * (teams + entries) +
// r + e: for one head group, r + e is unique because ranges and entries both advance with
// the position, and the slots of one (entry, head group) are consecutive in r, i.e. in
// token order.
struct Ranges {
    int T, n;
    __device__ int begin(int r) const { return r >= n ? T : (int)((int64_t)r * T / n); }
    __device__ int end(int r) const { return begin(r + 1); }
    // the r with begin(r) <= pos < end(r), for 0 <= pos < T
    __device__ int range_of(int pos) const { return (int)((((int64_t)pos + 1) * n - 1) / T); }
};

// Shared-prefix groups write 16-row partials, so their ranges are at least this long
// (short ranges cost more in partials and per-range start-up than they gain in waves).
constexpr int kMinGroupRange = 16;

__device__ Ranges make_ranges(const DecodeParams& p, int T) {
    Ranges r;
    r.T = T;
    r.n = p.teams < T ? p.teams : T;        // no empty range: a unit's ranges are consecutive
    if (p.sgroup > 0 && T / kMinGroupRange < r.n) r.n = T / kMinGroupRange;
    if (r.n < 1) r.n = 1;
    return r;
}

// Streams logical blocks [jb, je) of one sequence through NB register buffers of STEP
// blocks each: consume(j, buf) runs for blocks j .. j + STEP - 1 in order while the loads
// of the next NB-1 buffers are in flight.  Every issue is unconditional (the compiler can then count
// the loads and wait exactly for the oldest buffer): an issue for a block past the end
// of the current 64-block chunk loads through an empty buffer descriptor, which
// returns zeros without touching memory, and is never consumed.  The page table is
// read 64 ids at a time, one per lane (`tbl`, refreshed by table_chunk);
// issue(j, jend, jbase, buf) gets the chunk's end so it can tell live blocks apart.
template <int NB, int STEP, typename Buf, typename TableFn, typename IssueFn, typename ConsumeFn>
__device__ __forceinline__ void stream_blocks(int jb, int je, int& tbl, TableFn table_chunk, IssueFn issue,
                                              ConsumeFn consume) {
    static_assert(kWave % STEP == 0, "a buffer's blocks come from one table chunk");
    Buf buf[NB];
    bool ok[NB];
    for (int jc = jb; jc < je; jc += kWave) {
        if (jc != jb) tbl = table_chunk(jc);
        const int jend = min(je, jc + kWave);
#pragma unroll
        for (int k = 0; k < NB - 1; ++k) ok[k] = issue(jc + STEP * k, jend, jc, buf[k]);
        for (int j = jc; j < jend; j += NB * STEP) {
#pragma unroll
            for (int k = 0; k < NB; ++k) {
                const int nk = (k + NB - 1) % NB;
                ok[nk] = issue(j + STEP * (k + NB - 1), jend, jc, buf[nk]);
                if (j + STEP * k < jend && ok[k]) consume(j + STEP * k, buf[k]);
            }
        }
    }
}

// Physical block of logical block j (< jend) from the chunk held in `tbl`; -1 when j is
// past the end or the table entry is outside the pool.
__device__ __forceinline__ int live_block(const DecodeParams& p, int tbl, int j, int jend, int jbase) {
    const int phys = __builtin_amdgcn_readlane(tbl, (j < jend ? j : jend - 1) - jbase);
    return (j < jend && phys >= 0 && phys < p.num_blocks) ? phys : -1;
}

template <int N> struct Bytes;
template <> struct Bytes<4> { using T = uint32_t; };
template <> struct Bytes<8> { using T = uint2; };
template <> struct Bytes<16> { using T = uint4; };

template <typename W>
__device__ __forceinline__ void words_of(const W& w, uint32_t* out);
template <>
__device__ __forceinline__ void words_of<uint32_t>(const uint32_t& w, uint32_t* out) { out[0] = w; }
template <>
__device__ __forceinline__ void words_of<uint2>(const uint2& w, uint32_t* out) { out[0] = w.x; out[1] = w.y; }
template <>
__device__ __forceinline__ void words_of<uint4>(const uint4& w, uint32_t* out) {
    out[0] = w.x; out[1] = w.y; out[2] = w.z; out[3] = w.w;
}

template <typename W>
__device__ __forceinline__ W of_words(const uint32_t* w);
template <>
__device__ __forceinline__ uint32_t of_words<uint32_t>(const uint32_t* w) { return w[0]; }
template <>
__device__ __forceinline__ uint2 of_words<uint2>(const uint32_t* w) { return uint2{w[0], w[1]}; }
template <>
__device__ __forceinline__ uint4 of_words<uint4>(const uint32_t* w) { return uint4{w[0], w[1], w[2], w[3]}; }

// One segment of a wave's range in the balanced split: blocks [jb, je) of sequence (or
// group) b, jfirst .. nblk - 1 the blocks in play, lo the first token read, L the length
// (0 for groups), the workspace slot of its partial and whether that partial waits in the
// stash.
struct SegInfo {
    int b, jb, je, jfirst, nblk, lo, L;
    int64_t slot;
    bool defer;
};

// Fused append (pa_decode_append, 16-bit caches).  The new token of sequence b sits at
// position L - 1 of its last block; its K/V rows (new_key[b], new_value[b]: [Hkv, D], the
// cache dtype) replace, in registers, what a wave loads from that slot, and the lanes that
// hold those rows store them into the slot (one wave per (sequence, KV head)).  No wave reads
// the slot's old contents or depends on when the store lands.  The pieces are loaded when
// the segment starts and used only at its last block, so the loads wait for nothing.
struct NewToken {
    int o;      // offset of the token in its block
    int jnew;   // logical block holding the token

    static __device__ NewToken at(int L, int nblk) { return NewToken{(L - 1) % kBlockSize, nblk - 1}; }

    // Address of byte `byte` of the new row of sequence b, KV head hk (K or V).
    static __device__ const char* row(const void* base, const DecodeParams& p, int b, int hk, int D, int byte) {
        return (const char*)base + (((int64_t)b * p.Hkv + hk) * D) * 2 + byte;
    }

    // Where a lane's piece of the new row goes in the cache (K or V pool), or null when the
    // token's block is outside the pool.
    static __device__ char* slot_row(void* pool, const DecodeParams& p, int b, int hk, int D, int jnew, int o,
                                     int byte) {
        const int phys = p.block_tables[(int64_t)b * p.max_blocks + jnew];
        if (phys < 0 || phys >= p.num_blocks) return nullptr;
        return (char*)pool + (((int64_t)phys * kBlockSize + o) * p.Hkv + hk) * D * 2 + byte;
    }
};

// VALU path (head groups of 1, 2, 4 or 8 query heads).  One segment: blocks [jb, je) of
// sequence b (nblk blocks, L tokens), head group hg.  Writes the output rows when the
// segment is the whole sequence, else the partial for workspace slot `slot` (HPW
// consecutive heads per slot).
template <typename QT, typename CT, int D, int HPW, int NB, bool APPEND>
struct ValuSegment {
static constexpr int kWavesPerSimd = 1;   // no bound beyond the launch bounds
struct Buf {
    uint4 k[Layout<CT, D>::LPB], v[Layout<CT, D>::LPB];
    float ks[Layout<CT, D>::LPB], vs[Layout<CT, D>::LPB];
};
// Partials are stored where they are produced (defer is ignored; nothing to flush).
static __device__ __forceinline__ void flush(const DecodeParams&, int, int64_t) {}

// What a segment needs before it can issue its first block: the page-table chunk of block
// jb (lane i: the physical id of block jb + i).  Loaded one segment ahead, so a new segment
// starts its loads without waiting on memory (its queries load alongside its first block).
struct Pre {
    int tbl;
};
static __device__ __forceinline__ Pre prefetch(const DecodeParams& p, int lane, int b, int /*hg*/, int jb) {
    const int j = jb + lane;
    return Pre{j < p.max_blocks ? p.block_tables[(int64_t)b * p.max_blocks + j] : -1};
}

static __device__ __forceinline__ void run(const DecodeParams& p, int lane, int b, int hg, int jb, int je,
                                           int jfirst, int nblk, int lo, int L, int64_t slot, bool /*defer*/,
                                           const Pre& pre) {
    using Ly = Layout<CT, D>;
    constexpr int EB = Ly::EB, EPL = Ly::EPL, TPL = Ly::TPL, ROWS = Ly::ROWS, LPB = Ly::LPB;
    constexpr bool kFp8 = EB == 1;

    const int32_t* table = p.block_tables + (int64_t)b * p.max_blocks;
    // Page-table chunk: lane i holds the physical id of logical block jbase + i.
    auto table_chunk = [&](int jbase) {
        const int j = jbase + lane;
        return j < p.max_blocks ? table[j] : -1;
    };
    int tbl = pre.tbl;

    const int h0 = hg * HPW;
    const int hk = h0 / (p.Hq / p.Hkv);
    const int row = lane / TPL;
    const int chunk = lane % TPL;

    // Fused append: the segment that reads the sequence's last block loads this lane's 16 bytes
    // of the new token's rows; at that block the lanes of the token's row take them, and in the
    // first head group of each KV head also store them into the slot.
    static_assert(!(APPEND && kFp8), "the fused append covers 16-bit caches");
    NewToken nt{};
    uint4 knew{}, vnew{};
    const bool patch = APPEND && je == nblk && L > 0;
    if constexpr (APPEND) {
        if (patch) {
            nt = NewToken::at(L, nblk);
            knew = *(const uint4*)NewToken::row(p.new_key, p, b, hk, D, 16 * chunk);
            vnew = *(const uint4*)NewToken::row(p.new_value, p, b, hk, D, 16 * chunk);
        }
    }

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
    // physical id is lane j - jbase of `tbl`.  The K/V loads go through a descriptor of
    // the block (streaming: read once); past the chunk's end or for an id outside the pool
    // the descriptor is empty (zeros, no memory traffic) and the function returns false so
    // that the block is skipped.
    auto issue = [&](int j, int jend, int jbase, Buf& bf) {
        uint4(&kr)[LPB] = bf.k;
        uint4(&vr)[LPB] = bf.v;
        float(&ksc)[LPB] = bf.ks;
        float(&vsc)[LPB] = bf.vs;
        const int phys = live_block(p, tbl, j, jend, jbase);
        const bool ok = phys >= 0;
        const int64_t pb = ok ? phys : 0;
        const auto rk = block_rsrc(kbase + pb * blk_bytes, ok ? (int)blk_bytes : 0);
        const auto rv = block_rsrc(vbase + pb * blk_bytes, ok ? (int)blk_bytes : 0);
#pragma unroll
        for (int i = 0; i < LPB; ++i) kr[i] = buffer_load16<kCacheStream>(rk, lane_off + i * load_step);
#pragma unroll
        for (int i = 0; i < LPB; ++i) vr[i] = buffer_load16<kCacheStream>(rv, lane_off + i * load_step);
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
    auto consume = [&](int j, const Buf& bf) {
        uint4 kr[LPB], vr[LPB];
        float ksc[LPB], vsc[LPB];
#pragma unroll
        for (int i = 0; i < LPB; ++i) {
            kr[i] = bf.k[i];
            vr[i] = bf.v[i];
            ksc[i] = bf.ks[i];
            vsc[i] = bf.vs[i];
        }
        if constexpr (APPEND) {
            // the new token (row o of block jnew) comes from the inputs, not from its slot
            if (patch && j == nt.jnew) {
                const bool mine = row == nt.o % ROWS;
#pragma unroll
                for (int i = 0; i < LPB; ++i) {
                    if (i == nt.o / ROWS && mine) {
                        kr[i] = knew;
                        vr[i] = vnew;
                    }
                }
                if (mine && h0 % (p.Hq / p.Hkv) == 0) {
                    char* kd = NewToken::slot_row((void*)p.key_cache, p, b, hk, D, nt.jnew, nt.o, 16 * chunk);
                    char* vd = NewToken::slot_row((void*)p.value_cache, p, b, hk, D, nt.jnew, nt.o, 16 * chunk);
                    if (kd) {
                        *(uint4*)kd = knew;
                        *(uint4*)vd = vnew;
                    }
                }
            }
        }
        bool valid[LPB];
#pragma unroll
        for (int i = 0; i < LPB; ++i) {
            const int t = j * kBlockSize + i * ROWS + row;
            valid[i] = t >= lo && t < L;
        }

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

    stream_blocks<NB, 1, Buf>(jb, je, tbl, table_chunk, issue, consume);

    // Merge the ROWS row states (lanes with equal `chunk`); afterwards every row holds the
    // segment's result and the TPL lanes of row 0 write it.
    const bool whole = jb == jfirst && je == nblk;
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
};

// Matrix-core path for head groups of 3..16 query heads sharing one KV head (rows of
// a 16x16 tile; unused rows carry zero queries).  Per 16-token block, with lane l in
// row group g = l/16 and column c = l%16:
//   S^T[token][head] = K[token][:] . Q[head][:]   16x16x32 MFMAs over the head dim, K as
//       the A operand (lane l: token c), Q the B operand.  K is loaded in whole rows and
//       rearranged through a small per-wave LDS tile: loads that each cover a few full
//       rows stream faster than loads that each take a slice of all 16 rows.
//   online softmax per head on S^T (lane l: tokens 4g..4g+3 of head c), which is also the
//       A-operand layout of P in the next product.
//   O[head][col] += P[head][token] . V[token][col]   16x16x16 MFMAs, one per tile t < D/16;
//       V load i brings lane l the E = D/16 elements E c .. E c + E - 1 of token 4g + i,
//       and tile t's column n is head-dim index E n + t, so lane l's B operand for tile t
//       is element t of its four V loads: V reaches the matrix cores from registers.  P is
//       split into two operand-type terms (hi + lo), keeping ~16 more bits than one 16-bit
//       rounding.
// At the end lane l holds columns E c .. E c + E - 1 of heads 4g..4g+3 (contiguous stores).
// FP8 caches are widened to the query's 16-bit type (exactly) before the products; the
// per-token scales (four consecutive tokens per lane: one 16-byte load each for K and V)
// multiply the scores and P.

// Max and sum over the four 16-lane groups (lanes c, c + 16, c + 32, c + 48), every
// lane getting the result: gfx950's row and half-wave swaps, which stay in the VALU
// (a shuffle would make two round trips through the LDS crossbar).
__device__ __forceinline__ float group_max(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const float y = __builtin_fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
    return __builtin_fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float group_sum(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Slack of the matrix-core path's softmax reference (log2 units): exponentials up to
// 2^8 keep full relative precision in the hi + lo split and cannot overflow the fp32
// accumulators.
constexpr float kSlack = 8.0f;

// GROUPED: units of shared-prefix groups (rows = the group's sequences x heads); the
// ungrouped instantiation carries none of that code.
template <typename QT, typename CT, int D, int NB, bool GROUPED, bool APPEND>
struct MfmaSegment {
    using M = QT;
    static constexpr int EB = Storage<CT>::bytes;
    static constexpr bool kFp8 = EB == 1;
    // FP8 units run two waves per SIMD (the host launches twice the waves outside
    // shared-prefix groups), so their registers must fit in half the file.
    static constexpr int kWavesPerSimd = kFp8 ? 2 : 1;
    static constexpr int KSTEPS = D / 32;          // 16x16x32 steps over the head dimension
    static constexpr int E = D / 16;               // head-dim elements per lane per V row = tiles
    static constexpr int KLOADS = kFp8 ? KSTEPS / 2 : KSTEPS;   // 16-byte K loads per lane per block
    static constexpr int VBYTES = E * EB;          // V bytes per lane per row: 4, 8 or 16
    static constexpr int KLPR = D * EB / 16;       // lanes per K row in a whole-row load
    static constexpr int KTPL = kWave / KLPR;      // K rows per whole-row load
    static constexpr int KRS = D * EB + 16;        // LDS row stride (padded against bank conflicts)
    static_assert(KTPL * KLOADS == kBlockSize, "whole-row K loads cover the block");
    using VT = typename Bytes<VBYTES>::T;

    // FP8 scales: lane (g, c) holds the scale of token 4g + c % 4; each lane of a quad takes
    // the four of its lane group from the quad (quad_scale).
    struct Buf {
        uint4 k[KLOADS];
        VT v[4];
        float ks, vs;
    };
    // The ring holds blocks in pairs: the P V product runs on 16x16x32 tiles, whose 32-deep
    // contraction covers two blocks (k = 8 g + i is token 4 g + i % 4 of block i / 4; the
    // score tiles put exactly those tokens in lane group g).  ok[q]: block q is in the pool
    // and in the run (otherwise its loads returned zeros and its tokens are masked).
    struct Pair {
        Buf b[2];
        bool ok[2];
    };

    // B operand of tile t for one block: V rows 4g .. 4g + 3, element t of the lane's E,
    // as two words of operand-type pairs (rows 4g, 4g + 1 and rows 4g + 2, 4g + 3).
    // 16-bit: w[i][k] holds elements 2k, 2k + 1 of row i; one byte permute per word.
    static __device__ __forceinline__ uint2 v_tile16(const uint32_t (&w)[4][E / 2], int t) {
        const uint32_t sel = (t & 1) ? 0x07060302u : 0x05040100u;   // high or low halves of both
        const int k = t >> 1;
        return uint2{__builtin_amdgcn_perm(w[1][k], w[0][k], sel), __builtin_amdgcn_perm(w[3][k], w[2][k], sel)};
    }
    // FP8: x01[u][h] holds codes (row 0, row 1) of elements 4u + 2h and 4u + 2h + 1, byte
    // order r0, r1, r0, r1 (x23 the same for rows 2, 3), so one widening per word gives a pair.
    static __device__ __forceinline__ void v_codes(const uint32_t (&w)[4][(VBYTES + 3) / 4],
                                                   uint32_t (&x01)[(VBYTES + 3) / 4][2],
                                                   uint32_t (&x23)[(VBYTES + 3) / 4][2]) {
#pragma unroll
        for (int u = 0; u < (VBYTES + 3) / 4; ++u) {
            x01[u][0] = __builtin_amdgcn_perm(w[1][u], w[0][u], 0x05010400u);
            x01[u][1] = __builtin_amdgcn_perm(w[1][u], w[0][u], 0x07030602u);
            x23[u][0] = __builtin_amdgcn_perm(w[3][u], w[2][u], 0x05010400u);
            x23[u][1] = __builtin_amdgcn_perm(w[3][u], w[2][u], 0x07030602u);
        }
    }
    // (a plain DPP move: one instruction, with no zeroed destination to set up first)
    template <int R>
    static __device__ __forceinline__ float quad_scale(float x) {
        return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), R * 0x55, 0xF, 0xF, true));
    }
    static __device__ __forceinline__ uint32_t widen_sel(uint32_t x, int t) {
        return (t & 1) ? Mma<M>::template widen2<true>(x) : Mma<M>::template widen2<false>(x);
    }

    // Head-dimension index of element i (< 8) of MFMA step s for lane group g.  Any
    // mapping works as long as K and Q use the same one; these keep every lane's 16-byte
    // loads contiguous (FP8: one 16-byte load feeds two steps).
    static __device__ __forceinline__ int dk(int s, int g) {
        return kFp8 ? 64 * (s / 2) + 16 * g + 8 * (s % 2) : 32 * s + 8 * g;
    }

    // Eight FP8 codes (two words) -> eight operand-type values (exact), two per instruction.
    static __device__ __forceinline__ uint4 widen8(uint32_t w0, uint32_t w1) {
        return uint4{Mma<M>::template widen2<false>(w0), Mma<M>::template widen2<true>(w0),
                     Mma<M>::template widen2<false>(w1), Mma<M>::template widen2<true>(w1)};
    }

    // Unit u of sequence b: head group u / qgroups (G = hpw heads of one KV head) and query
    // group u % qgroups (qpw consecutive new tokens).  Row c < rows of the tile is query
    // c / G of the group and head c % G; with one query per sequence the rows are the heads.
    // One lane's V row piece (streaming load of VBYTES bytes).
    static __device__ __forceinline__ VT load_v(__amdgpu_buffer_rsrc_t r, uint32_t off) {
        if constexpr (VBYTES == 16) return buffer_load16<kCacheStream>(r, off);
        else if constexpr (VBYTES == 8) return buffer_load8<kCacheStream>(r, off);
        else return buffer_load4<kCacheStream>(r, off);
    }

    // A partial that is not the wave's last result (the wave's first segment, when the unit
    // began in an earlier range) waits in this wave's LDS stash and is written by flush()
    // after the wave's last segment.  Stores and loads share one completion counter that
    // retires in order, so a partial stored here would make the next segment's first loads
    // wait for the store to be acknowledged.  Per lane: O[t][r], m, the row total, a mask.
    static constexpr int kStash = 4 * E + 3;
    static __device__ __forceinline__ float* stash(int lane) {
        __shared__ float words[kWaves][kStash][kWave];
        return &words[__builtin_amdgcn_readfirstlane(threadIdx.x / kWave)][0][lane];
    }

    // The partial stores of a segment: rows 4g + r with bit r of `rows` set, (m, l) when bit 4.
    static __device__ __forceinline__ void store_partial(const DecodeParams& p, int lane, int64_t slot,
                                                         const f32x4_t* O, float m, float ltot, int rows) {
        const int c = lane & 15;
        const int g = lane >> 4;
        const int R = p.rows;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if (!((rows >> r) & 1)) continue;
            float4* arow = (float4*)(p.ws_acc + (slot * R + 4 * g + r) * D + E * c);
#pragma unroll
            for (int q = 0; q < E / 4; ++q)
                arow[q] = float4{O[4 * q][r], O[4 * q + 1][r], O[4 * q + 2][r], O[4 * q + 3][r]};
        }
        if ((rows >> 4) & 1) {
            p.ws_ml[(slot * R + c) * 2] = m;
            p.ws_ml[(slot * R + c) * 2 + 1] = ltot;
        }
    }

    // Writes the stashed partial to workspace slot `slot`.
    static __device__ __forceinline__ void flush(const DecodeParams& p, int lane, int64_t slot) {
        const float* st = stash(lane);
        f32x4_t O[E];
#pragma unroll
        for (int t = 0; t < E; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) O[t][r] = st[(4 * t + r) * kWave];
        store_partial(p, lane, slot, O, st[4 * E * kWave], st[(4 * E + 1) * kWave],
                      __float_as_int(st[(4 * E + 2) * kWave]));
    }

    // What a segment needs before it can issue its first block: the page-table chunk of
    // block jb (lane i: the physical id of block jb + i; groups load theirs per run).  Loaded
    // one segment ahead, so a new segment starts its loads without waiting on memory (its
    // queries load alongside its first blocks).
    struct Pre {
        int tbl;
    };
    static __device__ __forceinline__ Pre prefetch(const DecodeParams& p, int lane, int b, int /*u*/, int jb) {
        const int j = jb + lane;
        return Pre{(!GROUPED && j < p.max_blocks) ? p.block_tables[(int64_t)b * p.max_blocks + j] : -1};
    }

    static __device__ __forceinline__ void run(const DecodeParams& p, int lane, int b, int u, int jb, int je,
                                               int jfirst, int nblk, int lo, int L, int64_t slot, bool defer,
                                               const Pre& pre) {
        const int G = p.hpw;
        const int hg = u / p.qgroups;
        const int q0 = (u % p.qgroups) * p.qpw;        // first query of the unit
        const int h0 = hg * G;
        const int hk = h0 / (p.Hq / p.Hkv);
        const int c = lane & 15;
        const int g = lane >> 4;
        // Row of this lane's softmax column: its query, and the last token that query sees
        // (new token qi sits at position L - qlen + qi and attends to tokens up to there).
        // With shared-prefix groups the rows are the group's sequences b + qi instead (one
        // query each, attending to all of its L_qi tokens).
        constexpr bool grouped = GROUPED;
        const int qi = q0 + c / G;
        const bool row_ok = c < p.rows && qi < (grouped ? p.sgroup : p.qlen);
        // Groups: lane s < sgroup holds the length of the group's sequence s, lane sgroup the
        // group's prefix claim (one load for the wave).
        int glen = 0;
        if constexpr (grouped) {
            if (lane < p.sgroup) glen = seq_len(p, b + lane);
            else if (lane == p.sgroup) glen = p.prefix_blocks[b / p.sgroup];
        }
        const int rowL = grouped ? (row_ok ? __shfl(glen, qi) : 0) : L;
        const int last = grouped ? rowL - 1 : L - p.qlen + qi;

        // The blocks are streamed in runs, each from one page table with one set of rows
        // reading them: a single run for ungrouped units; for a group, the shared prefix
        // (every row) followed by each sequence's own blocks (that sequence's rows).
        // run_on: this lane's row reads the run; run_lv: tokens below it hold data that
        // some row of the run reads (V rows at or past it are zeroed).
        const int32_t* table = p.block_tables + (int64_t)b * p.max_blocks;
        bool run_on = true;
        int run_lv = L;
        auto table_chunk = [&](int jbase) {
            const int j = jbase + lane;
            return j < p.max_blocks ? table[j] : -1;
        };
        int tbl = pre.tbl;

        // Q as the B operand: lane l holds Q[row c][dk(s, g) + i]; zero for rows past the unit.
        uint4 qb[KSTEPS];
        {
            const int64_t qrow_idx = ((int64_t)b * p.qlen + (row_ok ? qi : 0)) * p.Hq + h0 + (row_ok ? c % G : 0);
            const uint16_t* qrow = (const uint16_t*)p.query + qrow_idx * D;
#pragma unroll
            for (int s = 0; s < KSTEPS; ++s) qb[s] = row_ok ? *(const uint4*)(qrow + dk(s, g)) : uint4{0u, 0u, 0u, 0u};
        }

        f32x4_t O[E];
#pragma unroll
        for (int t = 0; t < E; ++t) O[t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        float m = kNegInf;      // running max of head c (log2 units)
        float lsum = 0.0f;      // this lane's share of the running sum of head c

        const int64_t tok_bytes = (int64_t)p.Hkv * D * EB;
        const int64_t blk_bytes = tok_bytes * kBlockSize;
        const uint32_t v_off = (uint32_t)(4 * g * tok_bytes + (int64_t)hk * D * EB) + VBYTES * c;
        const uint32_t v_step = (uint32_t)tok_bytes;
        const char* kbase = (const char*)p.key_cache;
        const char* vbase = (const char*)p.value_cache;
        // K arrives in whole rows (lane l: 16 bytes at 16 (l % KLPR) of row KTPL i + l / KLPR)
        // and is turned into the operand layout through this wave's LDS tile.
        const uint32_t kr_off = (uint32_t)((lane / KLPR) * tok_bytes + (int64_t)hk * D * EB) + 16 * (lane % KLPR);
        // One tile per block of a pair.
        constexpr int TILE = kBlockSize * KRS;
        __shared__ uint4 ktiles[kWaves][2 * TILE / 16];
        char* ktile = (char*)ktiles[__builtin_amdgcn_readfirstlane(threadIdx.x / kWave)];
        char* kput = ktile + (lane / KLPR) * KRS + 16 * (lane % KLPR);
        const char* kget = ktile + c * KRS + 16 * g;

        // Fused append (ungrouped units of one query, 16-bit cache): the segment that reads the
        // sequence's last block loads this lane's pieces of the new token's rows (16 K bytes at the
        // lane's K column, VBYTES V bytes at its V column); at that block the lanes of the token's
        // row take them, and in the unit of the first heads of each KV head also store them.
        static_assert(!(APPEND && (GROUPED || kFp8)), "the fused append covers ungrouped 16-bit units");
        NewToken nt{};
        uint4 knew{};
        VT vnew{};
        const bool patch = APPEND && je == nblk && L > 0;
        if constexpr (APPEND) {
            if (patch) {
                nt = NewToken::at(L, nblk);
                knew = *(const uint4*)NewToken::row(p.new_key, p, b, hk, D, 16 * (lane % KLPR));
                vnew = *(const VT*)NewToken::row(p.new_value, p, b, hk, D, VBYTES * c);
            }
        }

        // Blocks j and j + 1 (K: KTPL whole rows per load.  V: rows 4g + i, E elements at E c.
        // Both are read once, in full lines, and streamed past the caches.)
        auto issue = [&](int j, int jend, int jbase, Pair& pr) {
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                Buf& bf = pr.b[q];
                const int phys = live_block(p, tbl, j + q, jend, jbase);
                const bool ok = phys >= 0;
                const int64_t pb = ok ? phys : 0;
                const auto rk = block_rsrc(kbase + pb * blk_bytes, ok ? (int)blk_bytes : 0);
                const auto rv = block_rsrc(vbase + pb * blk_bytes, ok ? (int)blk_bytes : 0);
#pragma unroll
                for (int i = 0; i < KLOADS; ++i)
                    bf.k[i] = buffer_load16<kCacheStream>(rk, kr_off + (uint32_t)(i * KTPL * tok_bytes));
#pragma unroll
                for (int i = 0; i < 4; ++i) bf.v[i] = load_v(rv, v_off + i * v_step);
                if constexpr (kFp8) {
                    bf.ks = p.k_scale[pb * kBlockSize + 4 * g + (lane & 3)];
                    bf.vs = p.v_scale[pb * kBlockSize + 4 * g + (lane & 3)];
                }
                pr.ok[q] = ok;
            }
            return pr.ok[0] || pr.ok[1];
        };

        // the new token (row o of block jnew) comes from the inputs, not from its slot
        auto patch_block = [&](Buf& bf) {
            const bool krow = lane / KLPR == nt.o % KTPL;
            const bool vrow = g == nt.o / 4;
#pragma unroll
            for (int i = 0; i < KLOADS; ++i)
                if (i == nt.o / KTPL && krow) bf.k[i] = knew;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (i == nt.o % 4 && vrow) bf.v[i] = vnew;
            if (h0 % (p.Hq / p.Hkv) == 0) {
                if (krow) {
                    char* kd = NewToken::slot_row((void*)p.key_cache, p, b, hk, D, nt.jnew, nt.o, 16 * (lane % KLPR));
                    if (kd) *(uint4*)kd = knew;
                }
                if (vrow) {
                    char* vd = NewToken::slot_row((void*)p.value_cache, p, b, hk, D, nt.jnew, nt.o, VBYTES * c);
                    if (vd) *(VT*)vd = vnew;
                }
            }
        };

        auto consume = [&](int j, const Pair& pr0) {
            Pair pr = pr0;
            if constexpr (APPEND) {
                if (patch && j == nt.jnew) patch_block(pr.b[0]);
                if (patch && j + 1 == nt.jnew) patch_block(pr.b[1]);
            }
            // K rows -> LDS -> A operand (lane l: 16 bytes of token c at byte 64 i + 16 g, i.e.
            // 16-bit step s = i, or FP8 steps 2i and 2i + 1).  The tiles belong to this wave
            // alone; the fences keep the compiler from moving these accesses past each other.
            uint4 ka[2][KLOADS];
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
            for (int q = 0; q < 2; ++q)
#pragma unroll
                for (int i = 0; i < KLOADS; ++i) *(uint4*)(kput + q * TILE + i * KTPL * KRS) = pr.b[q].k[i];
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
            for (int q = 0; q < 2; ++q)
#pragma unroll
                for (int i = 0; i < KLOADS; ++i) ka[q][i] = *(const uint4*)(kget + q * TILE + 64 * i);

            // S^T for each block's 16 tokens x 16 head rows (lane l: tokens 4g + r of head c).
            f32x4_t S[2];
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                S[q] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
                if constexpr (!kFp8) {
#pragma unroll
                    for (int s = 0; s < KSTEPS; ++s) S[q] = Mma<M>::k32(ka[q][s], qb[s], S[q]);
                } else {
#pragma unroll
                    for (int i = 0; i < KLOADS; ++i) {
                        S[q] = Mma<M>::k32(widen8(ka[q][i].x, ka[q][i].y), qb[2 * i], S[q]);
                        S[q] = Mma<M>::k32(widen8(ka[q][i].z, ka[q][i].w), qb[2 * i + 1], S[q]);
                    }
                }
            }
            // Score i < 8: token 4g + i % 4 of block i / 4, times the softmax scale (FP8: and the
            // token's K scale, this lane's one multiplied in before the quad shares them).
            float f[8];
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const float kl = kFp8 ? p.scale_log2 * pr.b[q].ks : p.scale_log2;
                f[4 * q + 0] = kFp8 ? quad_scale<0>(kl) : kl;
                f[4 * q + 1] = kFp8 ? quad_scale<1>(kl) : kl;
                f[4 * q + 2] = kFp8 ? quad_scale<2>(kl) : kl;
                f[4 * q + 3] = kFp8 ? quad_scale<3>(kl) : kl;
            }
            // (scaled unconditionally, then masked: a masked score is replaced whatever it holds)
            float sc[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) sc[i] = S[i / 4][i % 4] * f[i];
            // This lane's row attends to tokens [lo, hs).  The common case takes one test per
            // pair: both blocks hold data throughout and every row sees all of the pair or none
            // of it.  Otherwise, per token, valid: it holds data this unit reads (V rows of other
            // tokens select zeros); seen: this lane's row attends to it.
            const int j16 = j * kBlockSize;
            const int hs = run_on ? min(rowL, last + 1) : lo;
            const bool fast = pr.ok[0] && pr.ok[1] && j16 >= lo && j16 + 2 * kBlockSize <= run_lv &&
                              !__ballot(hs > j16 && hs < j16 + 2 * kBlockSize);
            bool valid[8], seen[8];
            if (fast) {
                const bool on = hs > j16;
#pragma unroll
                for (int i = 0; i < 8; ++i) sc[i] = on ? sc[i] : kNegInf;
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int t = j16 + kBlockSize * (i / 4) + 4 * g + i % 4;
                    valid[i] = pr.ok[i / 4] && t >= lo && t < run_lv;
                    seen[i] = valid[i] && run_on && t < rowL && t <= last;
                    sc[i] = seen[i] ? sc[i] : kNegInf;
                }
            }
            // Pair maximum of head c over the four lane groups.  The reference m moves only
            // when the pair exceeds it by more than kSlack (or on the first scores), so the
            // exponentials stay <= 2^kSlack and most pairs skip the output rescale; any
            // reference gives the same softmax, this one keeps the arithmetic in range.
            float mx = sc[0];
#pragma unroll
            for (int i = 1; i < 8; ++i) mx = __builtin_fmaxf(mx, sc[i]);
            const float mb = group_max(mx);
            const float mn = (mb > m + kSlack) ? mb : m;
            const float ms = (mn == kNegInf) ? 0.0f : mn;
            const float alpha = fast_exp2(m - ms);
            m = mn;
            float pw[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) pw[i] = fast_exp2(sc[i] - ms);
            float psum = pw[0];
#pragma unroll
            for (int i = 1; i < 8; ++i) psum += pw[i];
            if constexpr (kFp8) {
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const float vsc[4] = {quad_scale<0>(pr.b[q].vs), quad_scale<1>(pr.b[q].vs),
                                          quad_scale<2>(pr.b[q].vs), quad_scale<3>(pr.b[q].vs)};
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int i = 4 * q + r;
                        // (unwritten slots may hold any scale, even NaN: the product of an unseen
                        // token is replaced by zero)
                        pw[i] *= vsc[r];
                        if (!fast) pw[i] = seen[i] ? pw[i] : 0.0f;
                    }
                }
            }
            lsum = lsum * alpha + psum;
            // Rescale the output rows 4g + r when some running max moved.
            if (__ballot(alpha != 1.0f)) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float ar = __shfl(alpha, 4 * g + r);
#pragma unroll
                    for (int t = 0; t < E; ++t) O[t][r] *= ar;
                }
            }

            // P = hi + lo in the operand type (A operand: head c, k = 8g + i).
            uint32_t ph[4], pl[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                ph[k] = Mma<M>::pack_rtz(pw[2 * k], pw[2 * k + 1]);
                const float2_t fh = unpack2(M{}, ph[k]);
                pl[k] = Mma<M>::pack_rtz(pw[2 * k] - fh.x, pw[2 * k + 1] - fh.y);
            }
            const uint4 a_hi = uint4{ph[0], ph[1], ph[2], ph[3]};
            const uint4 a_lo = uint4{pl[0], pl[1], pl[2], pl[3]};

            // V of both blocks as B operands; rows past the data select zeros (P is zero there,
            // and 0 * NaN would not be).
            constexpr int VW = (VBYTES + 3) / 4;     // words per row piece
            uint32_t w[2][4][VW];
#pragma unroll
            for (int q = 0; q < 2; ++q)
#pragma unroll
                for (int i = 0; i < 4; ++i) words_of<VT>(pr.b[q].v[i], w[q][i]);
            if (!fast) {
#pragma unroll
                for (int q = 0; q < 2; ++q)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int u = 0; u < VW; ++u) w[q][i][u] = valid[4 * q + i] ? w[q][i][u] : 0u;
            }
            if constexpr (!kFp8) {
                static_assert(VW == E / 2, "16-bit rows: two elements per word");
#pragma unroll
                for (int t = 0; t < E; ++t) {
                    const uint2 b0 = v_tile16(w[0], t);
                    const uint2 b1 = v_tile16(w[1], t);
                    const uint4 bt = uint4{b0.x, b0.y, b1.x, b1.y};
                    O[t] = Mma<M>::k32(a_hi, bt, O[t]);
                    O[t] = Mma<M>::k32(a_lo, bt, O[t]);
                }
            } else {
                uint32_t x01[2][VW][2], x23[2][VW][2];
                v_codes(w[0], x01[0], x23[0]);
                v_codes(w[1], x01[1], x23[1]);
#pragma unroll
                for (int t = 0; t < E; ++t) {
                    const int u = t / 4, h = (t % 4) / 2;
                    const uint4 bt = uint4{widen_sel(x01[0][u][h], t), widen_sel(x23[0][u][h], t),
                                           widen_sel(x01[1][u][h], t), widen_sel(x23[1][u][h], t)};
                    O[t] = Mma<M>::k32(a_hi, bt, O[t]);
                    O[t] = Mma<M>::k32(a_lo, bt, O[t]);
                }
            }
        };

        // Group units: [jb, je) are positions in the unit's order, the prefix blocks 0 .. P-1
        // and then the blocks P .. n_s - 1 of each sequence s of the group in turn.
        int P = 0, lmax = 0;
        if constexpr (grouped) {
            int mn = 0x7fffffff;
            for (int s = 0; s < p.sgroup; ++s) {
                const int Ls = __builtin_amdgcn_readlane(glen, s);
                mn = min(mn, (Ls + kBlockSize - 1) / kBlockSize);
                lmax = max(lmax, Ls);
            }
            const int P0 = __builtin_amdgcn_readlane(glen, p.sgroup);
            P = P0 < 0 ? 0 : (P0 > mn ? mn : P0);
        }
        // One run per pass: its blocks [j0, j1), page table, rows and valid-token bound.
        for (int o = jb; o < je;) {
            int j0 = o, j1 = je;
            if constexpr (grouped) {
                if (o < P) {
                    j1 = min(P, je);
                    table = p.block_tables + (int64_t)b * p.max_blocks;
                    run_on = true;
                    run_lv = lmax;
                } else {
                    int base = P, s = 0, Ls = 0, n = 0;
                    for (; s < p.sgroup; ++s, base += n) {
                        Ls = __builtin_amdgcn_readlane(glen, s);
                        n = (Ls + kBlockSize - 1) / kBlockSize - P;
                        if (o < base + n) break;
                    }
                    if (s == p.sgroup) break;      // unreachable: positions end with the last sequence
                    j0 = P + (o - base);
                    j1 = P + min(n, je - base);
                    table = p.block_tables + (int64_t)(b + s) * p.max_blocks;
                    run_on = row_ok && qi == s;
                    run_lv = Ls;
                }
                tbl = table_chunk(j0);
            }
            stream_blocks<NB, 2, Pair>(j0, j1, tbl, table_chunk, issue, consume);
            o += j1 - j0;
        }

        // Totals per row (lane groups hold disjoint tokens), then per output row 4g + r.
        const float ltot = group_sum(lsum);
        const bool whole = jb == jfirst && je == nblk;
        const int R = p.rows;
        if (!whole) {
            int rows = (g == 0 && row_ok) ? 16 : 0;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 4 * g + r;
                if (row < R && q0 + row / G < (grouped ? p.sgroup : p.qlen)) rows |= 1 << r;
            }
            if (!defer) {
                store_partial(p, lane, slot, O, m, ltot, rows);
                return;
            }
            float* st = stash(lane);
#pragma unroll
            for (int t = 0; t < E; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) st[(4 * t + r) * kWave] = O[t][r];
            st[4 * E * kWave] = m;
            st[(4 * E + 1) * kWave] = ltot;
            st[(4 * E + 2) * kWave] = __int_as_float(rows);
            return;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 4 * g + r;
            const float lr = __shfl(ltot, row);
            const int rq = q0 + row / G;               // query (or group sequence) and head of this output row
            if (row >= R || rq >= (grouped ? p.sgroup : p.qlen)) continue;
            const int head = h0 + row % G;
            const float inv = lr > 0.0f ? 1.0f / lr : 0.0f;
            uint32_t packed[E / 2];
#pragma unroll
            for (int k = 0; k < E / 2; ++k)
                packed[k] = (uint32_t)to_bits(QT{}, O[2 * k][r] * inv) |
                            ((uint32_t)to_bits(QT{}, O[2 * k + 1][r] * inv) << 16);
            uint16_t* orow = (uint16_t*)p.out + (((int64_t)b * p.qlen + rq) * p.Hq + head) * D + E * c;
            if constexpr (E == 8) {
                *(uint4*)orow = uint4{packed[0], packed[1], packed[2], packed[3]};
            } else {
                *(uint2*)orow = uint2{packed[0], packed[1]};
            }
        }
    }
};


template <typename Segment>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(Segment::kWavesPerSimd)))
void decode_kernel(const DecodeParams p) {
    const int lane = threadIdx.x & (kWave - 1);
    const int w = blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    if (w >= p.num_waves) return;

    if (!p.balanced) {
        // Fixed partitions: wave w = (head group, partition, sequence), head group fastest, so
        // the waves of a team read one partition's blocks together.
        const int hg = w % p.groups;
        const int part = (w / p.groups) % p.NP;
        const int b = w / (p.groups * p.NP);
        const int s = b * p.groups + hg;
        // Partitions cover the blocks in play, j0 .. nblk - 1.
        const int L = seq_len(p, b);
        const int lo = first_token(p, L);
        const int j0 = lo / kBlockSize;
        const int nblk = (L + kBlockSize - 1) / kBlockSize;
        const int jb = j0 + part * p.part_blocks;
        if (jb >= nblk && !(part == 0 && nblk == 0)) return;   // L == 0: partition 0 writes zeros
        const int je = min(nblk, jb + p.part_blocks);
        Segment::run(p, lane, b, hg, jb, je, j0, nblk, lo, L, (int64_t)s * p.NP + part, false,
                     Segment::prefetch(p, lane, b, hg, jb));
        return;
    }

    // Balanced split: head group hg of the range of team `team` in the (sequence, block) order.
    // Workgroups go to the eight XCDs in turn (workgroup i on XCD i % 8); the waves are
    // renumbered so that each XCD holds one contiguous stretch of teams, i.e. neighbouring
    // positions (the beams of one prompt, whose shared blocks then meet in one L2).
    int wl = w;
    if (gridDim.x % 8 == 0 && p.num_waves == (int)gridDim.x * kWaves) {   // a permutation of the waves
        const int i = blockIdx.x;
        wl = ((i % 8) * (int)(gridDim.x / 8) + i / 8) * kWaves + (w - i * kWaves);
    }
    const int team = wl / p.groups;
    const int hg = wl % p.groups;
    Cursor cur = cursor_chunk(p, lane, 0, 0);
    const Ranges rg = make_ranges(p, num_entries(p) <= kWave ? cur.end : total_blocks(p, lane));
    // With fewer ranges than teams (little work, or the shared-prefix groups' minimum range
    // length) the ranges go to evenly spaced teams, so the idle teams spread over the XCDs:
    // team t runs range floor((t + 1) n / teams) - 1 when that differs from its predecessor's.
    const int r_next = (int)((int64_t)(team + 1) * rg.n / p.teams);
    if (r_next == (int)((int64_t)team * rg.n / p.teams)) return;
    const int r = r_next - 1;
    int pos = rg.begin(r);
    const int pos_end = rg.end(r);
    const int64_t slot_base = (int64_t)hg * (p.teams + num_entries(p)) + r;
    int64_t deferred = -1;   // workspace slot of a stashed partial
    // The range's segments in order; each one's table chunk and queries are loaded while the
    // one before it runs.
    auto next = [&](SegInfo& si) -> bool {
        if (pos >= pos_end) return false;
        // Position offsets count the blocks in play of the sequence, which start at logical
        // block jfirst.
        int len;
        const SeqPos sp = cursor_find(p, lane, cur, pos, len);
        // entry sp.b: a sequence, or the group of sequences sp.b * sgroup .. (whose segment
        // resolves its own lengths)
        si.b = p.sgroup > 0 ? sp.b * p.sgroup : sp.b;
        si.L = len;
        si.lo = first_token(p, len);
        si.jfirst = si.lo / kBlockSize;
        si.nblk = si.jfirst + sp.nblk;
        si.jb = si.jfirst + (pos - sp.start);
        si.je = min(si.nblk, si.jb + (pos_end - pos));
        si.slot = slot_base + sp.b;
        // Only a wave's first segment can end unfinished before its last one; its partial
        // is written after the last segment (see the segment's stash).
        const bool last = pos + (si.je - si.jb) >= pos_end;
        const bool whole = si.jb == si.jfirst && si.je == si.nblk;
        si.defer = !last;
        if (!last && !whole) deferred = si.slot;
        pos += si.je - si.jb;
        return true;
    };
    SegInfo si;
    bool has = next(si);
    typename Segment::Pre pre;
    if (has) pre = Segment::prefetch(p, lane, si.b, hg, si.jb);
    while (has) {
        SegInfo sn;
        const bool has_n = next(sn);
        typename Segment::Pre pre_n;
        if (has_n) pre_n = Segment::prefetch(p, lane, sn.b, hg, sn.jb);
        Segment::run(p, lane, si.b, hg, si.jb, si.je, si.jfirst, si.nblk, si.lo, si.L, si.slot, si.defer, pre);
        si = sn;
        pre = pre_n;
        has = has_n;
    }
    if (deferred >= 0) Segment::flush(p, lane, deferred);
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) x = __builtin_fmaxf(x, __shfl_xor(x, off));
    return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) x += __shfl_xor(x, off);
    return x;
}

// Merge of the partials of one output row (sequence, query, head), one wave each:
// out = sum_k 2^(m_k - M) acc_k / sum_k 2^(m_k - M) l_k over the segments of its
// unit in ascending token order (M = max_k m_k).  Lane k reads the (m, l)
// pair of partial k, so all pairs arrive in one round; the V sums are then
// folded in order k = 0, 1, ... with every lane holding D/64 columns.  Also
// writes the zero rows of empty sequences in the balanced split (no segment
// covers them).
template <typename QT, int D>
__global__ __launch_bounds__(kThreads) void decode_merge_kernel(const DecodeParams p) {
    constexpr int EPT = D / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t row = (int64_t)blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t per_seq = (int64_t)p.qlen * p.Hq;
    if (row >= (int64_t)p.B * per_seq) return;
    const int b = (int)(row / per_seq);
    const int h = (int)(row % per_seq) % p.Hq;
    // query (new token) of the row; with shared-prefix groups, the row's place in its group
    const int qi = p.sgroup > 0 ? b % p.sgroup : (int)(row % per_seq) / p.Hq;
    const int ent = p.sgroup > 0 ? b / p.sgroup : b;   // entry of the balanced order
    const int u = (h / p.hpw) * p.qgroups + qi / p.qpw;   // unit of (head group, query group)
    const int hh = (qi % p.qpw) * p.hpw + h % p.hpw;      // row within the unit's slots
    const int64_t s = (int64_t)ent * p.groups + u;
    uint16_t* orow = (uint16_t*)p.out + row * D;

    int64_t first;
    int count;
    if (!p.balanced) {
        const int nblk = seq_blocks(p, b);
        const int n_part = (nblk + p.part_blocks - 1) / p.part_blocks;
        if (n_part <= 1) return;            // written by the one partition (zeros when L == 0)
        first = s * p.NP;
        count = n_part;
    } else {
        const SeqTable st = seq_table(p, lane);
        const Ranges rg = make_ranges(p, st.total);
        const SeqPos e = seq_entry(p, st, lane, ent);
        if (e.nblk == 0) {
#pragma unroll
            for (int k = 0; k < EPT; ++k) orow[k * kWave + lane] = to_bits(QT{}, 0.0f);
            return;
        }
        const int t0 = rg.range_of(e.start);
        const int t1 = rg.range_of(e.start + e.nblk - 1);
        if (t0 == t1) return;               // one segment: written directly
        first = (int64_t)u * (p.teams + num_entries(p)) + t0 + ent;
        count = t1 - t0 + 1;
    }

    const int hpw = p.rows;                 // partial rows per slot
    const float* ml = p.ws_ml;
    const float* acc = p.ws_acc + (first * hpw + hh) * D + lane;   // partial k at acc[k * hpw * D]
    const int64_t kstride = (int64_t)hpw * D;

    // The V sums of the first kPre partials are loaded together with the (m, l) pairs.
    constexpr int kPre = 16;
    float pre[kPre][EPT];
#pragma unroll
    for (int k = 0; k < kPre; ++k)
#pragma unroll
        for (int e = 0; e < EPT; ++e) pre[k][e] = k < count ? acc[k * kstride + e * kWave] : 0.0f;

    float m0 = kNegInf, l0 = 0.0f;          // this lane's pair of the first 64 partials
    float M = kNegInf;
    for (int k0 = 0; k0 < count; k0 += kWave) {
        const int k = k0 + lane;
        float mk = kNegInf, lk = 0.0f;
        if (k < count) {
            const int64_t hs = (first + k) * hpw + hh;
            mk = ml[hs * 2];
            lk = ml[hs * 2 + 1];
        }
        if (k0 == 0) {
            m0 = mk;
            l0 = lk;
        }
        M = __builtin_fmaxf(M, wave_max(mk));
    }
    const float ms = (M == kNegInf) ? 0.0f : M;

    float num[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) num[e] = 0.0f;
    float den = 0.0f;
    for (int k0 = 0; k0 < count; k0 += kWave) {
        const int k = k0 + lane;
        float mk = m0, lk = l0;
        if (k0 > 0) {
            mk = kNegInf;
            lk = 0.0f;
            if (k < count) {
                const int64_t hs = (first + k) * hpw + hh;
                mk = ml[hs * 2];
                lk = ml[hs * 2 + 1];
            }
        }
        const float f = k < count ? fast_exp2(mk - ms) : 0.0f;
        den += wave_sum(f * lk);
        const int n = min(kWave, count - k0);
        int j = 0;
        if (k0 == 0) {
#pragma unroll
            for (; j < kPre; ++j) {
                if (j >= n) break;
                const float fj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), j));
#pragma unroll
                for (int e = 0; e < EPT; ++e) num[e] = __builtin_fmaf(fj, pre[j][e], num[e]);
            }
        }
#pragma unroll 8
        for (; j < n; ++j) {
            const float fj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), j));
#pragma unroll
            for (int e = 0; e < EPT; ++e) num[e] = __builtin_fmaf(fj, acc[(k0 + j) * kstride + e * kWave], num[e]);
        }
    }
#pragma unroll
    for (int e = 0; e < EPT; ++e) orow[e * kWave + lane] = to_bits(QT{}, den > 0.0f ? num[e] / den : 0.0f);
}

// Merge of long lists of fixed partitions (split-K over long contexts): one workgroup
// per output row.  Every wave computes the common maximum M and the denominator over
// all partials; wave w folds the V sums of the w-th contiguous quarter of the list,
// loading kBatch partials at a time; the quarters are added in order w = 0, 1, ...
// through LDS, so the result is deterministic for fixed inputs.
template <typename QT, int D>
__global__ __launch_bounds__(kThreads) void decode_merge_split_kernel(const DecodeParams p) {
    constexpr int EPT = D / kWave;
    constexpr int kBatch = 16;
    __shared__ float quarter[kWaves][D];
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t row = blockIdx.x;                 // grid = output rows
    const int64_t per_seq = (int64_t)p.qlen * p.Hq;
    const int b = (int)(row / per_seq);
    const int qi = (int)(row % per_seq) / p.Hq;
    const int h = (int)(row % per_seq) % p.Hq;
    const int u = (h / p.hpw) * p.qgroups + qi / p.qpw;
    const int hh = (qi % p.qpw) * p.hpw + h % p.hpw;
    const int64_t s = (int64_t)b * p.groups + u;
    const int nblk = seq_blocks(p, b);
    const int count = (nblk + p.part_blocks - 1) / p.part_blocks;
    if (count <= 1) return;                  // written by the one partition (the whole workgroup)
    const int64_t first = s * p.NP;
    const int hpw = p.rows;
    const float* ml = p.ws_ml;
    const float* acc = p.ws_acc + (first * hpw + hh) * D + lane;
    const int64_t kstride = (int64_t)hpw * D;
    auto pair = [&](int k, float& mk, float& lk) {
        mk = kNegInf;
        lk = 0.0f;
        if (k < count) {
            const int64_t hs = (first + k) * hpw + hh;
            mk = ml[hs * 2];
            lk = ml[hs * 2 + 1];
        }
    };

    float M = kNegInf;
    for (int k0 = 0; k0 < count; k0 += kWave) {
        float mk, lk;
        pair(k0 + lane, mk, lk);
        M = __builtin_fmaxf(M, wave_max(mk));
    }
    const float ms = (M == kNegInf) ? 0.0f : M;
    float den = 0.0f;
    for (int k0 = 0; k0 < count; k0 += kWave) {
        float mk, lk;
        pair(k0 + lane, mk, lk);
        den += wave_sum(k0 + lane < count ? fast_exp2(mk - ms) * lk : 0.0f);
    }

    const int q = (count + kWaves - 1) / kWaves;
    const int k_lo = min(count, wv * q), k_hi = min(count, k_lo + q);
    float num[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) num[e] = 0.0f;
    for (int k0 = k_lo; k0 < k_hi; k0 += kWave) {
        float mk, lk;
        pair(k0 + lane, mk, lk);
        const float f = k0 + lane < k_hi ? fast_exp2(mk - ms) : 0.0f;
        const int n = min(kWave, k_hi - k0);
        int j = 0;
#pragma unroll 1
        for (; j + kBatch <= n; j += kBatch) {
            float v[kBatch][EPT];
#pragma unroll
            for (int t = 0; t < kBatch; ++t)
#pragma unroll
                for (int e = 0; e < EPT; ++e) v[t][e] = acc[(k0 + j + t) * kstride + e * kWave];
#pragma unroll
            for (int t = 0; t < kBatch; ++t) {
                const float fj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), j + t));
#pragma unroll
                for (int e = 0; e < EPT; ++e) num[e] = __builtin_fmaf(fj, v[t][e], num[e]);
            }
        }
        for (; j < n; ++j) {
            const float fj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), j));
#pragma unroll
            for (int e = 0; e < EPT; ++e) num[e] = __builtin_fmaf(fj, acc[(k0 + j) * kstride + e * kWave], num[e]);
        }
    }
#pragma unroll
    for (int e = 0; e < EPT; ++e) quarter[wv][e * kWave + lane] = num[e];
    __syncthreads();
    if (wv != 0) return;
    uint16_t* orow = (uint16_t*)p.out + row * D;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        float t = quarter[0][e * kWave + lane];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) t += quarter[w][e * kWave + lane];
        orow[e * kWave + lane] = to_bits(QT{}, den > 0.0f ? t / den : 0.0f);
    }
}

// Fixed split-K with more partitions than this per sequence merges with the split kernel.
constexpr int kLongMerge = 48;

template <typename QT, int D, typename Segment>
hipError_t run(const DecodeParams& p, hipStream_t stream) {
    const int64_t grid = ((int64_t)p.num_waves + kWaves - 1) / kWaves;
    hipLaunchKernelGGL((decode_kernel<Segment>), dim3((uint32_t)grid), dim3(kThreads), 0, stream, p);
    if (p.balanced || p.NP > 1) {
        const int64_t rows = (int64_t)p.B * p.qlen * p.Hq;   // one merge wave per (sequence, query, head)
        if (!p.balanced && p.NP > kLongMerge)
            hipLaunchKernelGGL((decode_merge_split_kernel<QT, D>), dim3((uint32_t)rows), dim3(kThreads), 0, stream, p);
        else
            hipLaunchKernelGGL((decode_merge_kernel<QT, D>), dim3((uint32_t)((rows + kWaves - 1) / kWaves)),
                               dim3(kThreads), 0, stream, p);
    }
    return hipGetLastError();
}

// Two blocks in flight per wave: deeper rings measured no faster.
constexpr int kRing = 2;

// APPEND: kernels of the fused append + decode (one query per sequence, no shared-prefix groups).
template <typename QT, typename CT, int D, bool APPEND>
hipError_t run_path(const DecodeParams& p, hipStream_t s) {
    if (p.mfma) {
        if constexpr (!APPEND) {
            if (p.sgroup > 0) return run<QT, D, MfmaSegment<QT, CT, D, kRing, true, false>>(p, s);
        }
        return run<QT, D, MfmaSegment<QT, CT, D, kRing, false, APPEND>>(p, s);
    }
    switch (p.hpw) {
        case 1: return run<QT, D, ValuSegment<QT, CT, D, 1, kRing, APPEND>>(p, s);
        case 2: return run<QT, D, ValuSegment<QT, CT, D, 2, kRing, APPEND>>(p, s);
        case 4: return run<QT, D, ValuSegment<QT, CT, D, 4, kRing, APPEND>>(p, s);
        case 8: return run<QT, D, ValuSegment<QT, CT, D, 8, kRing, APPEND>>(p, s);
        default: return hipErrorInvalidValue;
    }
}

template <typename QT, typename CT, bool APPEND>
hipError_t run_d(const DecodeParams& p, int d, hipStream_t s) {
    switch (d) {
        case 64: return run_path<QT, CT, 64, APPEND>(p, s);
        case 128: return run_path<QT, CT, 128, APPEND>(p, s);
        default: return hipErrorInvalidValue;
    }
}

// The fused append covers 16-bit caches; an FP8 cache's append runs as its own kernel (the
// per-token scale needs the whole token before any code is known).
template <bool APPEND>
hipError_t launch(const DecodeParams& p, int head_dim, int q_kind, int cache_kind, hipStream_t stream) {
    if (q_kind == kF16 && cache_kind == kF16) return run_d<F16, F16, APPEND>(p, head_dim, stream);
    if (q_kind == kBF16 && cache_kind == kBF16) return run_d<BF16, BF16, APPEND>(p, head_dim, stream);
    if constexpr (!APPEND) {
        if (q_kind == kF16 && cache_kind == kFP8) return run_d<F16, FP8, false>(p, head_dim, stream);
        if (q_kind == kBF16 && cache_kind == kFP8) return run_d<BF16, FP8, false>(p, head_dim, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace

// This source is compiled twice: once for the plain decode kernels (PA_DECODE_APPEND unset)
// and once for the fused append + decode kernels, so the two sets build in parallel.
#if PA_DECODE_APPEND
hipError_t launch_decode_append(const DecodeParams& p, int head_dim, int q_kind, int cache_kind,
                                hipStream_t stream) {
    return launch<true>(p, head_dim, q_kind, cache_kind, stream);
}
#else
HeadGrouping head_grouping(int group) {
    // Groups of 3 to 16 heads (or multiples of 16) go to the matrix cores, padded to 16
    // rows; smaller groups stay on the VALU path.
    if (group % 16 == 0) return {16, true};
    if (group >= 3 && group <= 16) return {group, true};
    for (int h = 8; h > 1; h >>= 1)
        if (group % h == 0) return {h, false};
    return {1, false};
}

HeadGrouping multi_query_grouping(int group) {
    // Several queries per sequence always take the matrix cores: a unit holds the heads of
    // one KV head (up to 16; larger groups split into the largest divisor <= 16) and as
    // many of the sequence's queries as fill the 16 rows.
    if (group <= 16) return {group, true};
    for (int h = 16; h > 1; --h)
        if (group % h == 0) return {h, true};
    return {1, true};
}

hipError_t launch_decode(const DecodeParams& p, int head_dim, int q_kind, int cache_kind, hipStream_t stream) {
    return launch<false>(p, head_dim, q_kind, cache_kind, stream);
}
#endif

}  // namespace pa
