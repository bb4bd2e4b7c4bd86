// Exact GQA attention of the step's query over the attended token set T.
//
// Source: page "KV Cache 与长上下文推理", section "KV Cache 回顾": the decode
// attention softmax(q K^T / sqrt(d_k)) V, here restricted to T (kept chunks
// plus sink and window); the GQA table of section "KV Cache 压缩技术" maps
// query head h to KV head h / G.  The score matrix is never written to
// memory: each split keeps a running max, a running sum and an fp32
// accumulator (the tiling idea the InfiniteHiP article credits to
// FlashAttention, section "从赫赫有名的注意力机制说起"), and the last split
// of each (request, KV head) to finish merges all splits by log-sum-exp.
//
// Workgroup (split, request, KV head) = 4 waves: the last nsplit_a splits
// take the sink and window (dispatched last, so that their bulk loads queue
// behind the other splits' small loads of the select inputs); the others
// select the last stage's kept set themselves (fused plan: the last two
// stages), or read it from kept_idx when the stage is reused, and take the
// kept chunks' blocks (with values in host memory, the value-cache kernel's
// block list instead); waves take the split's blocks round-robin.  For one 8-token
// block a wave computes the G scores of every token (lane = token * 8 +
// 16-dim slice; bf16 pair dot products, DPP sum over the 8 slice lanes),
// takes the block max per head (uniform over the wave), then accumulates
// P V with lane l owning output dims 2l and 2l+1, reading each value row
// with one coalesced dword per lane; where a wave takes more than one pair
// of blocks, the running max and the rescale are taken once per pair.  All
// splits of a (request, KV head) run on one XCD (sd_device.h), so the merge
// reads their partials from its L2.
#include "sd_device.h"
#include "sd_internal.h"
#include "sd_select.h"

namespace sd {

constexpr int kAttnThreads = 256;
constexpr int kAttnWaves = kAttnThreads / kWave;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

struct AttendParams {
    const uint16_t* q;        // [B][Hq][d]
    const uint16_t* k;        // [B][Hkv][Lmax][d]
    const uint16_t* v;        // [B][Hkv][Lmax][d] values (device, or the device alias of pinned host memory)
    uint16_t* vpool;          // [B][Hkv][slots][8][d] (host-value path)
    const int32_t* blk_slot;  // [B][Hkv][max_blocks]   (host-value path)
    int vslots;
    int vcopied;              // host values: this step's missed blocks were copied into their slots already
    const int32_t* lengths;
    const uint32_t* blocks;   // [B][Hkv][max_blocks] (host-value path: built by the value-cache kernel)
    const int32_t* nblocks;   // [B][Hkv]           (host-value path)
    int max_blocks;
    // last-stage select (device-value path)
    StageDev last;
    int first_stage;          // the last stage is also the first
    int pp_koff;              // kept_idx offset of the stage before the last
    int32_t* last_scores;     // [B][Hkv][last.ncand] (fused: written here, for inspection)
    // fused last two stages: P = the stage before the last
    StageDev P;
    int p_first;              // P is the first stage
    int pp_koff_p;            // kept_idx offset of the stage before P
    const int32_t* p_scores;  // [B][Hkv][P.ncand]
    const int32_t* pre;       // [B][Hkv][P.ncand * fuse_rq] every child's last-stage score
    int fuse_rq;
    int32_t* kept;            // [B][Hkv][keep_total]
    int keep_total;
    int32_t* flag;            // error flags; a bad length is flagged here when the last stage is given
    int sink, window;
    float* part;              // acc [B*Hkv][nsplit][G][d], then (m, l) [B*Hkv][nsplit][G][2]
    int nsplit;               // splits per (request, KV head)
    int nsplit_a;             // of which sink/window splits (device values)
    int Bh;                   // B * Hkv
    int32_t* tick;            // [B*Hkv][kTickInts] hand-off counters (merge by the last split)
    int64_t Lmax;
    int Hq, Hkv;
    float scale_log2;
    uint16_t* out;            // [B][Hq][d]
    uint32_t* rec;            // null, or [B][Hkv][max_blocks]: the (block << 8 | mask) words attended
};

__device__ __forceinline__ float dot2bf(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                           false);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// exp2(a - m) with exp2(-inf - m) = 0 and no NaN when both are -inf.
__device__ __forceinline__ float rescale(float a, float m) {
    return a == -INFINITY ? 0.0f : fast_exp2(a - m);
}

// Token positions fit 32 bits (max_context < 2^31 - 8 is checked at
// creation), so block and mask arithmetic is 32-bit.
//
// Tokens of block blk below L.
__device__ __forceinline__ uint32_t valid_mask8(int blk, int L) {
    const int over = blk * 8 + 8 - L;
    return over <= 0 ? 0xffu : over >= 8 ? 0u : (0xffu >> over);
}
// Tokens of block blk in the sink [0, s_end) or the window [w0, L).
__device__ __forceinline__ uint32_t sinkwin_mask8(int blk, int L, int s_end, int w0) {
    const int lo = min(max(s_end - blk * 8, 0), 8);   // tokens below s_end
    const int hi = min(max(w0 - blk * 8, 0), 8);      // first token at or after w0
    const uint32_t m = ((1u << lo) - 1u) | (0xffu & (0xffu << hi));
    return m & valid_mask8(blk, L);
}

// Where a workgroup's blocks come from (one kind per workgroup, so each
// kind gets its own copy of the block loop).
//  ListSrc:  the block list built by the value-cache kernel (host values)
//  RangeSrc: the sink and window ranges, masked to sink/window tokens
//  KeptSrc:  the kept last-stage chunks' blocks, masked to the tokens the
//            ranges do not cover (the two masks are disjoint; their union is T)
struct ListSrc {
    const uint32_t* list;
    __device__ void at(int r, int& blk, uint32_t& mask) const {
        const uint32_t e = list[r];
        blk = int(e >> 8);
        mask = e & 0xffu;
    }
};
struct RangeSrc {
    int nr1, wb0, s_end, w0, L;
    __device__ void at(int r, int& blk, uint32_t& mask) const {
        blk = r < nr1 ? r : wb0 + (r - nr1);
        mask = sinkwin_mask8(blk, L, s_end, w0);
    }
};
struct KeptSrc {
    const int* kept;            // LDS, ascending kept starts
    int bpc, s_end, w0, L;
    __device__ void at(int r, int& blk, uint32_t& mask) const {
        const int q = r / bpc;
        blk = (kept[q] >> 3) + (r - q * bpc);
        mask = valid_mask8(blk, L) & ~sinkwin_mask8(blk, L, s_end, w0);
    }
};

struct BlockData {
    u32x4 k0, k1;
    uint32_t vv[8];
    uint32_t mask;
};

// Loads of one block (t0 = first token, mask = tokens that count).  Device
// values: every load is issued unconditionally, from rows clamped below L
// (always inside the cache), and rows outside the mask are zeroed by a
// select, so the issue is branch-free.  Host values: hits come from the slot
// pool, misses and refills from host memory (rows t < L), written into their
// slot.  KROWS = false: the values only (the keys come by load_pair_k).
template <bool HOSTV, bool KROWS = true>
__device__ __forceinline__ void load_block(const AttendParams& p, int r, int t0, uint32_t mask, int bj, int L,
                                           const uint16_t* kbase, const uint16_t* vbase, BlockData& d) {
    const int lane = threadIdx.x & 63, tok = lane >> 3, sl = lane & 7;
    d.mask = mask;
    if constexpr (KROWS) {
        const u32x4* kp = reinterpret_cast<const u32x4*>(kbase + int64_t(min(t0 + tok, L - 1)) * kHeadDim + sl * 16);
        d.k0 = __builtin_nontemporal_load(kp);
        d.k1 = __builtin_nontemporal_load(kp + 1);
    }
    if (HOSTV) {
        const int32_t se = p.blk_slot[int64_t(bj) * p.max_blocks + r];
        uint32_t* prow = reinterpret_cast<uint32_t*>(p.vpool + (int64_t(bj) * p.vslots + (se & kVcSlotMask)) * 8 * kHeadDim);
        if (!p.vcopied && (se & (kVcMissBit | kVcRefillBit))) {
            const uint32_t* hrow = reinterpret_cast<const uint32_t*>(vbase + int64_t(t0) * kHeadDim);
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                d.vv[u] = (t0 + u < L) ? hrow[u * (kHeadDim / 2) + lane] : 0u;
                if (t0 + u < L) prow[u * (kHeadDim / 2) + lane] = d.vv[u];
            }
        } else {
#pragma unroll
            for (int u = 0; u < 8; ++u) d.vv[u] = ((mask >> u) & 1u) ? prow[u * (kHeadDim / 2) + lane] : 0u;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) d.vv[u] = ((mask >> u) & 1u) ? d.vv[u] : 0u;
    } else {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const uint32_t* vrow = reinterpret_cast<const uint32_t*>(vbase + int64_t(min(t0 + u, L - 1)) * kHeadDim);
            d.vv[u] = __builtin_nontemporal_load(vrow + lane);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) d.vv[u] = ((mask >> u) & 1u) ? d.vv[u] : 0u;
    }
}

// G = 4 on the matrix cores.  The scores of a pair of blocks (16 tokens)
// for the group's 4 query heads are one 16 x 16 x 128 product, four
// v_mfma_f32_16x16x32_bf16 (bf16 products, fp32 sums): A = the 16 key rows
// (lane l: token row l % 16 of the pair, block (l % 16) / 8), B = the query
// (lane l: head l % 16 of the group, clamped to the group's last for
// l % 16 >= 4, whose columns are never read).  Instruction i takes dims
// 32 i + 8 c + e, e < 8, from lane group c = l / 16, for A and B alike, so
// the four cover each dim once and one instruction's key loads stay inside
// one 64-byte piece of each row (one cache line per row).  The result leaves lane l holding tokens
// 4 c + r, r < 4, of head l % 16: each lane keeps the running max and its
// share of the sum for its head, and the heads' softmax runs side by side.
// P V stays on the vector ALU (lane l owns dims 2l, 2l+1, as in
// attend_block).
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Max or sum of lane l's value and lane (l ^ 16)'s (or (l ^ 32)'s), by the
// row-swap permutes (no LDS round trip): swapping a register with itself
// leaves lane l's own value in one result and its partner's in the other,
// so a symmetric operation on the two gives the pair's.
__device__ __forceinline__ float max_xor16_f(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32_f(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16_f(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32_f(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

struct PairK {
    u32x4 k[4];
};

// The A operand of a pair's keys: blocks at t0a and t0b (t0b = t0a when
// the pair has one block; its tokens are masked), rows clamped below L.
__device__ __forceinline__ void load_pair_k(int t0a, int t0b, int L, const uint16_t* kbase, PairK& pk) {
    const int lane = threadIdx.x & 63, m = lane & 15, c = lane >> 4;
    const int t = min((m < 8 ? t0a : t0b) + (m & 7), L - 1);
    const u32x4* kp = reinterpret_cast<const u32x4*>(kbase + int64_t(t) * kHeadDim + 8 * c);
#pragma unroll
    for (int i = 0; i < 4; ++i) pk.k[i] = __builtin_nontemporal_load(kp + 4 * i);
}

// Running max of head lane % 16 (the same in its four lanes) and this
// lane's share of that head's sum (its tokens 4 (lane / 16) + r).
struct MState {
    float m, l;
};

// Online-softmax update with a pair of blocks on the matrix cores; d1's
// values are read only when `two` (else its tokens count for nothing).
__device__ __forceinline__ void attend_pair_mfma(const PairK& pk, const BlockData& d0, const BlockData& d1, bool two,
                                                 const u32x4 (&qb)[4], float scale_log2, MState& st,
                                                 float (&acc0)[4], float (&acc1)[4]) {
    const int lane = threadIdx.x & 63;
    f32x4_t d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i)
        d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, pk.k[i]),
                                                    __builtin_bit_cast(bf16x8_t, qb[i]), d, 0, 0, 0);
    const int t0 = 4 * (lane >> 4);                     // this lane's first token of the 16
    const uint32_t mask1 = two ? d1.mask : 0u;
    const uint32_t msk = t0 < 8 ? (d0.mask >> t0) : (mask1 >> (t0 - 8));
    float z[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) z[r] = ((msk >> r) & 1u) ? d[r] * scale_log2 : -INFINITY;
    float bm = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
    bm = max_xor32_f(max_xor16_f(bm));                  // the head's other token groups
    const float mn = fmaxf(st.m, bm);
    const float alpha = rescale(st.m, mn);
    float pw[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) pw[r] = ((msk >> r) & 1u) ? fast_exp2(z[r] - mn) : 0.f;
    st.l = st.l * alpha + ((pw[0] + pw[1]) + (pw[2] + pw[3]));
    st.m = mn;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), h));
        acc0[h] *= a;
        acc1[h] *= a;
    }
    // tokens outside the masks have p = 0 and zeroed values: no branch
#pragma unroll
    for (int t = 0; t < 16; ++t) {
        const uint32_t w = t < 8 ? d0.vv[t] : (two ? d1.vv[t - 8] : 0u);
        const float v0 = bf16_lo(w), v1 = bf16_hi(w);
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            const float pu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pw[t & 3]), h + 16 * (t >> 2)));
            acc0[h] = fmaf(pu, v0, acc0[h]);
            acc1[h] = fmaf(pu, v1, acc1[h]);
        }
    }
}

// Online-softmax update of one wave's state with one block.
template <int G>
__device__ __forceinline__ void attend_block(const BlockData& d, const uint32_t (&qv)[G][8], float scale_log2,
                                             float (&m)[G], float (&lsum)[G], float (&acc0)[G], float (&acc1)[G]) {
    const int lane = threadIdx.x & 63, tok = lane >> 3;
    const bool in = (d.mask >> tok) & 1u;
    float z[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        float s = dot2bf(qv[h][0], d.k0.x, 0.f);
        s = dot2bf(qv[h][1], d.k0.y, s);
        s = dot2bf(qv[h][2], d.k0.z, s);
        s = dot2bf(qv[h][3], d.k0.w, s);
        s = dot2bf(qv[h][4], d.k1.x, s);
        s = dot2bf(qv[h][5], d.k1.y, s);
        s = dot2bf(qv[h][6], d.k1.z, s);
        s = dot2bf(qv[h][7], d.k1.w, s);
        s = sum8_f(s);
        z[h] = in ? s * scale_log2 : -INFINITY;
    }
    float pw[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const float bm = max_groups_f(z[h]);
        const float mn = fmaxf(m[h], bm);
        const float alpha = rescale(m[h], mn);
        pw[h] = in ? fast_exp2(z[h] - mn) : 0.f;
        lsum[h] = lsum[h] * alpha + pw[h];
        acc0[h] *= alpha;
        acc1[h] *= alpha;
        m[h] = mn;
    }
    // tokens outside the mask have p = 0 and zeroed values: no branch
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const float v0 = bf16_lo(d.vv[u]), v1 = bf16_hi(d.vv[u]);
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float pu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pw[h]), u * 8));
            acc0[h] = fmaf(pu, v0, acc0[h]);
            acc1[h] = fmaf(pu, v1, acc1[h]);
        }
    }
}

// The same update with two blocks at once (16 tokens): the running max,
// the rescale of the state and its exp2 are taken once for the pair.
// ORDERED (blocks whose loads were just issued): the first block's scores,
// then the second's, and the first block's values before the second's, with
// scheduling barriers between them, so that the wave starts on the first
// block as soon as its rows arrive (its loads were issued first).  Not
// ORDERED (rows loaded long before): the two blocks' chains interleave.
template <int G, bool ORDERED>
__device__ __forceinline__ void attend_pair(const BlockData& d0, const BlockData& d1, const uint32_t (&qv)[G][8],
                                            float scale_log2, float (&m)[G], float (&lsum)[G], float (&acc0)[G],
                                            float (&acc1)[G]) {
    const int lane = threadIdx.x & 63, tok = lane >> 3;
    const bool in0 = (d0.mask >> tok) & 1u, in1 = (d1.mask >> tok) & 1u;
    auto score = [&](const BlockData& d, int h) {
        float s = dot2bf(qv[h][0], d.k0.x, 0.f);
        s = dot2bf(qv[h][1], d.k0.y, s);
        s = dot2bf(qv[h][2], d.k0.z, s);
        s = dot2bf(qv[h][3], d.k0.w, s);
        s = dot2bf(qv[h][4], d.k1.x, s);
        s = dot2bf(qv[h][5], d.k1.y, s);
        s = dot2bf(qv[h][6], d.k1.z, s);
        s = dot2bf(qv[h][7], d.k1.w, s);
        return sum8_f(s);
    };
    float z0[G], z1[G];
#pragma unroll
    for (int h = 0; h < G; ++h) z0[h] = in0 ? score(d0, h) * scale_log2 : -INFINITY;
    if constexpr (ORDERED) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int h = 0; h < G; ++h) z1[h] = in1 ? score(d1, h) * scale_log2 : -INFINITY;
    float pw0[G], pw1[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const float bm = max_groups_f(fmaxf(z0[h], z1[h]));
        const float mn = fmaxf(m[h], bm);
        const float alpha = rescale(m[h], mn);
        pw0[h] = in0 ? fast_exp2(z0[h] - mn) : 0.f;
        pw1[h] = in1 ? fast_exp2(z1[h] - mn) : 0.f;
        lsum[h] = lsum[h] * alpha + (pw0[h] + pw1[h]);
        acc0[h] *= alpha;
        acc1[h] *= alpha;
        m[h] = mn;
    }
    auto pv = [&](const BlockData& d, const float (&pw)[G]) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const float v0 = bf16_lo(d.vv[u]), v1 = bf16_hi(d.vv[u]);
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float pu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pw[h]), u * 8));
                acc0[h] = fmaf(pu, v0, acc0[h]);
                acc1[h] = fmaf(pu, v1, acc1[h]);
            }
        }
    };
    pv(d0, pw0);
    if constexpr (ORDERED) __builtin_amdgcn_sched_barrier(0);
    pv(d1, pw1);
}

// The block loop of one workgroup over blocks [r0, r1) of its source.  The
// (block, mask) entries are computed once per tile of kBlkTile blocks, one
// per thread, into LDS (and, when rec is not null, stored as rec[r] =
// block << 8 | mask for inspection); each wave then takes every
// kAttnWaves-th block of the tile, two blocks in flight.
constexpr int kBlkTile = kAttnThreads;

template <int G, bool HOSTV, bool MF, class Src>
__device__ __forceinline__ void decode_blocks(const AttendParams& p, const Src& src, int r0, int r1, int bj, int L,
                                              const uint16_t* kbase, const uint16_t* vbase,
                                              const uint32_t (&qv)[G][8], const uint16_t* qg, float (&m)[G],
                                              float (&lsum)[G], float (&acc0)[G], float (&acc1)[G], int* tblk,
                                              uint32_t* tmask, uint32_t* rec) {
    const int wave = threadIdx.x >> 6;
    if (L <= 0) return;                    // no blocks (and no row to clamp to)
    // MF (the wide decode, G = 4) and more than one pair per wave: pairs of
    // blocks on the matrix cores (a last single block as a pair whose second
    // half is masked).  The one-request plans' splits are latency-bound (a
    // wave waits for a pair's rows, then has little left to compute); they
    // take the vector path below, which starts on each block as its rows
    // arrive and measured faster there.
    if constexpr (MF && G == 4) if (r1 - r0 > 2 * kAttnWaves) {
        // the query as the B operand: lane l gives head l % 16 (clamped to
        // the group's last head; those columns are never read)
        u32x4 qb[4];
        {
            const int lane = threadIdx.x & 63;
            const u32x4* qp = reinterpret_cast<const u32x4*>(qg + min(lane & 15, G - 1) * kHeadDim + 8 * (lane >> 4));
#pragma unroll
            for (int i = 0; i < 4; ++i) qb[i] = qp[4 * i];
        }
        MState st{-INFINITY, 0.f};
        for (int tb = r0; tb < r1; tb += kBlkTile) {
            const int n = min(kBlkTile, r1 - tb);
            if (int(threadIdx.x) < n) {
                int blk;
                uint32_t mask;
                src.at(tb + threadIdx.x, blk, mask);
                tblk[threadIdx.x] = blk * 8;
                tmask[threadIdx.x] = mask;
                if (rec) rec[tb + threadIdx.x] = (uint32_t(blk) << 8) | mask;
            }
            __syncthreads();
            for (int i = wave; i < n; i += 2 * kAttnWaves) {
                BlockData d0, d1;
                PairK pk;
                const bool two = i + kAttnWaves < n;
                const int i1 = two ? i + kAttnWaves : i;
                load_pair_k(tblk[i], tblk[i1], L, kbase, pk);
                load_block<HOSTV, false>(p, tb + i, tblk[i], tmask[i], bj, L, kbase, vbase, d0);
                if (two) load_block<HOSTV, false>(p, tb + i1, tblk[i1], tmask[i1], bj, L, kbase, vbase, d1);
                attend_pair_mfma(pk, d0, d1, two, qb, p.scale_log2, st, acc0, acc1);
            }
            __syncthreads();
        }
        // to the per-head state of the vector path: the max, and the sum in
        // lane 0 only (write_partials adds one lane per 8-lane token group)
        const float x = sum_xor32_f(sum_xor16_f(st.l));
        const int lane = threadIdx.x & 63;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            m[h] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(st.m), h));
            const float tot = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), h));
            lsum[h] = lane == 0 ? tot : 0.f;
        }
        return;
    }
    for (int tb = r0; tb < r1; tb += kBlkTile) {
        const int n = min(kBlkTile, r1 - tb);
        if (int(threadIdx.x) < n) {
            int blk;
            uint32_t mask;
            src.at(tb + threadIdx.x, blk, mask);
            tblk[threadIdx.x] = blk * 8;
            tmask[threadIdx.x] = mask;
            if (rec) rec[tb + threadIdx.x] = (uint32_t(blk) << 8) | mask;
        }
        __syncthreads();
        for (int i = wave; i < n; i += 2 * kAttnWaves) {
            BlockData d0, d1;
            const bool two = i + kAttnWaves < n;
            load_block<HOSTV>(p, tb + i, tblk[i], tmask[i], bj, L, kbase, vbase, d0);
            if (two) load_block<HOSTV>(p, tb + i + kAttnWaves, tblk[i + kAttnWaves], tmask[i + kAttnWaves], bj, L, kbase,
                                       vbase, d1);
            if (two && n > 2 * kAttnWaves) {
                // more than one pair per wave: one softmax update per pair
                attend_pair<G, true>(d0, d1, qv, p.scale_log2, m, lsum, acc0, acc1);
            } else {
                // at most a pair per wave (a latency-bound split): each
                // block as soon as its rows arrive
                attend_block<G>(d0, qv, p.scale_log2, m, lsum, acc0, acc1);
                if (two) attend_block<G>(d1, qv, p.scale_log2, m, lsum, acc0, acc1);
            }
        }
        __syncthreads();
    }
}

// Merges the four waves' online-softmax states of one workgroup and stores
// them as split `sp` of (request, KV head) bj: acc at [bj][sp][h][dd] (one
// contiguous G x 128 slab per workgroup), (m, l) at [bj][sp][h][2] after
// all acc (nsplit splits per (request, KV head)).
template <int G>
__device__ __forceinline__ void write_partials(float* part, int Bh, int nsplit, int bj, int sp, const float (&m)[G],
                                               const float (&lsum)[G], const float (&acc0)[G], const float (&acc1)[G],
                                               float (&wm)[kAttnWaves][G], float (&wl)[kAttnWaves][G],
                                               float (&wacc)[kAttnWaves][G][kHeadDim]) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // wave totals: lsum is per token group (identical in its 8 lanes)
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const float lt = sum_groups_f(lsum[h]);
        if (lane == 0) { wm[wave][h] = m[h]; wl[wave][h] = lt; }
        wacc[wave][h][2 * lane] = acc0[h];
        wacc[wave][h][2 * lane + 1] = acc1[h];
    }
    __syncthreads();
    float* pacc = part + (int64_t(bj) * nsplit + sp) * G * kHeadDim;
    float* pml = part + int64_t(Bh) * G * kHeadDim * nsplit + (int64_t(bj) * nsplit + sp) * G * 2;
    for (int o = threadIdx.x; o < G * kHeadDim; o += kAttnThreads) {
        const int h = o / kHeadDim, dd = o % kHeadDim;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kAttnWaves; ++w) M = fmaxf(M, wm[w][h]);
        float a = 0.f, l = 0.f;
#pragma unroll
        for (int w = 0; w < kAttnWaves; ++w) {
            const float f = rescale(wm[w][h], M);
            a = fmaf(wacc[w][h][dd], f, a);
            l = fmaf(wl[w][h], f, l);
        }
        pacc[o] = a;
        if (dd == 0) {
            pml[h * 2] = M;
            pml[h * 2 + 1] = l;
        }
    }
}

// Log-sum-exp merge of the nsplit partials of (request, KV head) bj into
// the bf16 output of its G query heads, by the last split to finish (its
// partials were written in this launch on the same XCD: read from the L2).
// Weights exp2(m_s - M) / sum_s l_s exp2(m_s - M) per head (wave h < G,
// lane = split); thread t sums output quad t % (32 G) over the splits
// t / (32 G) + k SG (SG = 8 / G split groups, every float4 load issued at
// once: one memory round trip), and the split groups are added through LDS.
// MAXS: the most splits the launch can have (kDecodeMaxSplits, or
// kDecodeWideSplits for the wide kernel); it sizes the per-thread loads,
// the kernel's largest register set.
template <int G, int MAXS>
__device__ __forceinline__ void merge_splits(const AttendParams& p, int bj, int b, int j, float* wgt, float4* red) {
    static_assert(MAXS <= kDecodeMaxSplits, "one split per lane in the weight pass");
    constexpr int NQ = G * kHeadDim / 4;         // float4 quads of outputs
    constexpr int SG = kAttnThreads / NQ;        // split groups
    constexpr int NB = (MAXS + SG - 1) / SG;     // splits per thread, at most
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int q = tid % NQ, sg = tid / NQ, h = (4 * q) / kHeadDim;
    const int ns = p.nsplit;
    const float* pa = p.part + int64_t(bj) * ns * G * kHeadDim + 4 * q;
    const float* pml = p.part + int64_t(p.Bh) * G * kHeadDim * ns + int64_t(bj) * ns * G * 2;
    // every load issued at once (splits beyond ns re-read the last one; their weight is 0)
    float4 v[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u)
        v[u] = *reinterpret_cast<const float4*>(pa + int64_t(min(sg + u * SG, ns - 1)) * G * kHeadDim);
    if (wave < G) {
        const float2 ml = *reinterpret_cast<const float2*>(pml + min(lane, ns - 1) * G * 2 + wave * 2);
        const float m = lane < ns ? ml.x : -INFINITY;
        const float l = lane < ns ? ml.y : 0.f;
        const float M = wave_max_f(m);
        const float f = rescale(m, M);
        const float Lt = wave_sum_f(l * f);
        wgt[wave * kWave + lane] = (lane < ns && Lt > 0.f) ? f / Lt : 0.f;
    }
    __syncthreads();
    SD_PHASE(3, 7);
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int u = 0; u < NB; ++u) {
        const int sp = sg + u * SG;
        const float wv = sp < ns ? wgt[h * kWave + sp] : 0.f;
        a.x = fmaf(v[u].x, wv, a.x);
        a.y = fmaf(v[u].y, wv, a.y);
        a.z = fmaf(v[u].z, wv, a.z);
        a.w = fmaf(v[u].w, wv, a.w);
    }
    red[sg * NQ + q] = a;
    __syncthreads();
    if (tid < NQ) {
        float4 t = red[tid];
#pragma unroll
        for (int g = 1; g < SG; ++g) {
            const float4 u = red[g * NQ + tid];
            t.x += u.x;
            t.y += u.y;
            t.z += u.z;
            t.w += u.w;
        }
        const int hh = (4 * tid) / kHeadDim, dd = (4 * tid) % kHeadDim;
        uint16_t* o = p.out + (int64_t(b) * p.Hq + j * G + hh) * kHeadDim + dd;
        const uint32_t lo = uint32_t(f32_to_bf16_rne(t.x)) | (uint32_t(f32_to_bf16_rne(t.y)) << 16);
        const uint32_t hi = uint32_t(f32_to_bf16_rne(t.z)) | (uint32_t(f32_to_bf16_rne(t.w)) << 16);
        *reinterpret_cast<uint2*>(o) = make_uint2(lo, hi);
    }
}

// One instantiation per (group size, values on host, select code of the
// last stage (kGiven: reused, read from kept_idx; unused with host values),
// select code of the stage before it when the last two stages are fused
// here (0 = not fused)).
//
// Workgroup slots follow pipe_slot (all splits of a (request, KV head) on
// one XCD): the kept-chunk splits come first, the sink/window splits last.
// Every kept-chunk split selects the last stage's kept set itself (the
// selection is deterministic, so they agree) and the first of them
// publishes it to kept_idx; the last split to finish merges all partials.
template <int G, bool HOSTV, int SEL, int SELP, int MAXS = kDecodeMaxSplits>
__global__ __launch_bounds__(kAttnThreads) void sd_flash_decode_kernel(AttendParams p) {
    extern __shared__ uint32_t dyn[];   // device values: the select (keys, sel, scratch)
    __shared__ float wm[kAttnWaves][G];
    __shared__ float wl[kAttnWaves][G];
    __shared__ float wacc[kAttnWaves][G][kHeadDim];
    __shared__ unsigned tmp[32];
    __shared__ int tblk[kBlkTile];          // first token of each block of the current tile
    __shared__ uint32_t tmask[kBlkTile];    // its token mask
    __shared__ int ticket;
    __shared__ float4 red[kAttnThreads];    // the merge's reduction over split groups
    static_assert(sizeof(tblk) >= sizeof(float) * 4 * kWave, "the merge's weights fit the block tile");

    SD_PHASE(3, 0);
    const PipeSlot ps = pipe_slot(p.nsplit, p.Bh);
    if (ps.bj < 0) return;
    const int bj = ps.bj, sp = ps.w;
    const int b = bj / p.Hkv, j = bj - b * p.Hkv;
    const int lane = threadIdx.x & 63;
    const int sl = lane & 7;
    // the length, sanitised where each path first needs it (the kept-chunk
    // splits' select loads do not wait for it)
    const int32_t Lraw = load_length(p.lengths, b);
    auto length = [&]() -> int { return int(length_here(Lraw, p.Lmax)); };

    // this lane's 16 query dims of every head of the group (bf16 pairs)
    uint32_t qv[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const u32x4* qp = reinterpret_cast<const u32x4*>(p.q + (int64_t(b) * p.Hq + j * G + h) * kHeadDim + sl * 16);
        const u32x4 a = qp[0], c = qp[1];
        qv[h][0] = a.x; qv[h][1] = a.y; qv[h][2] = a.z; qv[h][3] = a.w;
        qv[h][4] = c.x; qv[h][5] = c.y; qv[h][6] = c.z; qv[h][7] = c.w;
    }

    // the group's query rows (the matrix-core path loads its own operand)
    const uint16_t* qg = p.q + (int64_t(b) * p.Hq + j * G) * kHeadDim;

    float m[G], lsum[G], acc0[G], acc1[G];
#pragma unroll
    for (int h = 0; h < G; ++h) { m[h] = -INFINITY; lsum[h] = 0.f; acc0[h] = 0.f; acc1[h] = 0.f; }

    const uint16_t* kbase = p.k + int64_t(bj) * p.Lmax * kHeadDim;
    const uint16_t* vbase = p.v + int64_t(bj) * p.Lmax * kHeadDim;

    // inspection record of this pipeline's attended words: host values, the
    // block list; device values, the kept blocks, then (from kept_words on)
    // the sink / window blocks
    uint32_t* rec = p.rec ? p.rec + int64_t(bj) * p.max_blocks : nullptr;
    const int kept_words = p.last.keep * (p.last.chunk >> 3);

    int kept_n = -1;
    FusedOut fused{};
    if (HOSTV) {
        const int L = length();
        const int nb = p.nblocks[bj];
        const int per = (nb + p.nsplit - 1) / p.nsplit;
        const int r0 = min(nb, sp * per), r1 = min(nb, r0 + per);
        decode_blocks<G, HOSTV, !HOSTV && MAXS == kDecodeWideSplits>(p, ListSrc{p.blocks + int64_t(bj) * p.max_blocks}, r0, r1, bj, L, kbase, vbase,
                                qv, qg, m, lsum, acc0, acc1, tblk, tmask, rec);
    } else if (sp >= p.nsplit - p.nsplit_a) {
        // sink / window blocks: known without any selection
        const int L = length();
        const int s_end = min(p.sink, L);
        const int w0 = p.window > 0 ? max(0, L - p.window) : L;
        const int sb1 = (s_end + 7) >> 3, wb1 = (L + 7) >> 3;
        const int wb0 = p.window > 0 ? (w0 >> 3) : wb1;
        const bool merged = wb0 <= sb1;
        const int nr1 = merged ? wb1 : sb1;
        const int nb = nr1 + (merged ? 0 : wb1 - wb0);
        const int per = (nb + p.nsplit_a - 1) / p.nsplit_a;
        const int spa = sp - (p.nsplit - p.nsplit_a);
        const int r0 = min(nb, spa * per), r1 = min(nb, r0 + per);
        decode_blocks<G, HOSTV, !HOSTV && MAXS == kDecodeWideSplits>(p, RangeSrc{nr1, wb0, s_end, w0, L}, r0, r1, bj, L, kbase, vbase, qv, qg, m, lsum,
                                acc0, acc1, tblk, tmask, rec ? rec + kept_words : nullptr);
    } else {
        // the kept chunks of the last stage, recomputed from its scores
        // (fused: from the previous stage's scores and every child's
        // precomputed score)
        int32_t* kept_bj = p.kept + int64_t(bj) * p.keep_total;
        int nk;
        const int* kstarts;
        // (the selects take Lmax as the length bound: a selected candidate
        // has a score, so it starts below the length anyway)
        if constexpr (SEL == kGiven) {
            // the last stage is reused: its kept set is read from kept_idx
            // (and no pruning kernel ran this step to flag a bad length)
            const int Lg = length();
            if (Lg == 0 && sp == 0 && threadIdx.x == 0) atomicOr(p.flag, kFlagBadLength);
            int* sel = reinterpret_cast<int*>(dyn + p.last.ncand);
            nk = given_kept<kAttnThreads>(p.last, kept_bj + p.last.koff, Lg, sel, tmp);
            kstarts = sel;
        } else if constexpr (SELP != 0) {
            const FusedOut fo = kept_two_stages<kAttnThreads, SELP, SEL>(
                p.P, p.p_first != 0, p.p_scores + int64_t(bj) * p.P.ncand, p.p_first ? nullptr : kept_bj + p.pp_koff_p,
                p.pre + int64_t(bj) * p.P.ncand * p.fuse_rq, p.fuse_rq, p.last, p.Lmax, dyn, tmp);
            nk = fo.nq;
            kstarts = fo.q_starts;
            fused = fo;
        } else {
            nk = kept_of_stage<kAttnThreads, SEL>(p.last, p.first_stage != 0, p.last_scores + int64_t(bj) * p.last.ncand,
                                                  p.first_stage ? nullptr : kept_bj + p.pp_koff, p.Lmax, dyn, tmp);
            kstarts = reinterpret_cast<const int*>(dyn + p.last.ncand);
        }
        const int L = length();
        SD_PHASE(3, 2);
        kept_n = sp == 0 && SEL != kGiven ? nk : -1;   // the first of these workgroups publishes the kept set
        const int s_end = min(p.sink, L);
        const int w0 = p.window > 0 ? max(0, L - p.window) : L;
        const int nsb = p.nsplit - p.nsplit_a;
        const int bpc = p.last.chunk >> 3;
        const int nb = nk * bpc;
        const int per = (nb + nsb - 1) / nsb;
        const int r0 = min(nb, sp * per), r1 = min(nb, r0 + per);
        decode_blocks<G, HOSTV, !HOSTV && MAXS == kDecodeWideSplits>(p, KeptSrc{kstarts, bpc, s_end, w0, L}, r0, r1, bj, L, kbase, vbase, qv, qg, m, lsum,
                                acc0, acc1, tblk, tmask, rec);
    }

    SD_PHASE(3, 3);
    write_partials<G>(p.part, p.Bh, p.nsplit, bj, sp, m, lsum, acc0, acc1, wm, wl, wacc);
    if (!HOSTV && kept_n >= 0) {
        // the last stage's kept set (ascending, -1 padded); fused: also the
        // previous stage's kept set and the last stage's candidate scores
        int32_t* kept_bj = p.kept + int64_t(bj) * p.keep_total;
        const int* sel = SELP != 0 ? fused.q_starts : reinterpret_cast<const int*>(dyn + p.last.ncand);
        for (int i = threadIdx.x; i < p.last.keep; i += kAttnThreads) kept_bj[p.last.koff + i] = i < kept_n ? sel[i] : -1;
        if (SELP != 0) {
            for (int i = threadIdx.x; i < p.P.keep; i += kAttnThreads) kept_bj[p.P.koff + i] = fused.p_starts[i];
            int32_t* sc = p.last_scores + int64_t(bj) * p.last.ncand;
            for (int i = threadIdx.x; i < p.last.ncand; i += kAttnThreads) {
                const uint32_t key = fused.q_keys[i];
                sc[i] = key ? int32_t(key) - (1 << 23) : INT32_MIN;
            }
        }
    }
    SD_PHASE(3, 4);
    // the last split of this (request, KV head) to finish merges them all
    const bool last = handoff_last(p.tick + int64_t(bj) * kTickInts, p.nsplit, &ticket, p.flag);
    SD_PHASE(3, 5);
    if (!last) return;
    merge_splits<G, MAXS>(p, bj, b, j, reinterpret_cast<float*>(tblk), red);
    SD_PHASE(3, 6);
}

// Dense decode over every token t < L, the comparison path of
// sd_dense_decode.  Workgroup (split, KV head, request) takes a contiguous
// run of 8-token blocks; wave w takes blocks w, w + 4, w + 8, ... of the run
// and keeps four blocks in flight: it issues the loads of the next pair
// before it attends the current pair, so the block loop never waits on a
// load issued in the same iteration.  Loads, scores and the online softmax
// are the sparse decode's (load_block, attend_block); only the block source
// differs (every block, masked to t < L).
template <int G>
__global__ __launch_bounds__(kAttnThreads) void sd_dense_decode_kernel(AttendParams p) {
    __shared__ float wm[kAttnWaves][G];
    __shared__ float wl[kAttnWaves][G];
    __shared__ float wacc[kAttnWaves][G][kHeadDim];

    const int sp = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
    const int bj = b * p.Hkv + j;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int sl = lane & 7;
    const int32_t Lraw = load_length(p.lengths, b);
    const bool bad = Lraw < 1 || Lraw > p.Lmax;
    const int L = bad ? 0 : int(Lraw);
    if (bad && sp == 0 && j == 0 && threadIdx.x == 0) atomicOr(p.flag, 1);

    uint32_t qv[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const u32x4* qp = reinterpret_cast<const u32x4*>(p.q + (int64_t(b) * p.Hq + j * G + h) * kHeadDim + sl * 16);
        const u32x4 a = qp[0], c = qp[1];
        qv[h][0] = a.x; qv[h][1] = a.y; qv[h][2] = a.z; qv[h][3] = a.w;
        qv[h][4] = c.x; qv[h][5] = c.y; qv[h][6] = c.z; qv[h][7] = c.w;
    }
    float m[G], lsum[G], acc0[G], acc1[G];
#pragma unroll
    for (int h = 0; h < G; ++h) { m[h] = -INFINITY; lsum[h] = 0.f; acc0[h] = 0.f; acc1[h] = 0.f; }

    const uint16_t* kbase = p.k + int64_t(bj) * p.Lmax * kHeadDim;
    const uint16_t* vbase = p.v + int64_t(bj) * p.Lmax * kHeadDim;
    const int nb = (L + 7) >> 3;
    // whole groups of 2 x 4 blocks per split, so every wave gets pairs
    constexpr int kGrp = 2 * kAttnWaves;
    const int per = ((nb + p.nsplit - 1) / p.nsplit + kGrp - 1) / kGrp * kGrp;
    const int r0 = min(nb, sp * per), r1 = min(nb, r0 + per);

    // wave-uniform block indices; a block at or past r1 is neither loaded nor attended
    int r = r0 + wave;
    BlockData a0, a1, b0, b1;
    if (r < r1) load_block<false>(p, r, r * 8, valid_mask8(r, L), bj, L, kbase, vbase, a0);
    if (r + kAttnWaves < r1)
        load_block<false>(p, r + kAttnWaves, (r + kAttnWaves) * 8, valid_mask8(r + kAttnWaves, L), bj, L, kbase,
                          vbase, a1);
    for (; r < r1; r += 2 * kGrp) {
        const int rb = r + kGrp;
        if (rb < r1) load_block<false>(p, rb, rb * 8, valid_mask8(rb, L), bj, L, kbase, vbase, b0);
        if (rb + kAttnWaves < r1)
            load_block<false>(p, rb + kAttnWaves, (rb + kAttnWaves) * 8, valid_mask8(rb + kAttnWaves, L), bj, L,
                              kbase, vbase, b1);
        if (r + kAttnWaves < r1) attend_pair<G, false>(a0, a1, qv, p.scale_log2, m, lsum, acc0, acc1);
        else attend_block<G>(a0, qv, p.scale_log2, m, lsum, acc0, acc1);
        if (rb >= r1) break;
        const int ra = rb + kGrp;
        if (ra < r1) load_block<false>(p, ra, ra * 8, valid_mask8(ra, L), bj, L, kbase, vbase, a0);
        if (ra + kAttnWaves < r1)
            load_block<false>(p, ra + kAttnWaves, (ra + kAttnWaves) * 8, valid_mask8(ra + kAttnWaves, L), bj, L,
                              kbase, vbase, a1);
        if (rb + kAttnWaves < r1) attend_pair<G, false>(b0, b1, qv, p.scale_log2, m, lsum, acc0, acc1);
        else attend_block<G>(b0, qv, p.scale_log2, m, lsum, acc0, acc1);
    }
    write_partials<G>(p.part, p.Bh, p.nsplit, bj, sp, m, lsum, acc0, acc1, wm, wl, wacc);
}

// Log-sum-exp merge of the splits, rounding to bf16.  A workgroup merges 64
// outputs of one head: thread t reads float4 q = t % 16 of those outputs from
// splits t / 16, t / 16 + 16, ... (each split's 64 values are one contiguous
// 256 B row, so the reads coalesce).  The partial loads are issued first;
// wave 0 meanwhile computes the head's split weights
// exp2(m_s - M) / sum_s l_s exp2(m_s - M); each thread sums its splits
// weighted, and the 16 split groups are added through LDS.
// MAXS is the largest split count an instantiation merges: 64 for the
// sparse decode (one split per lane of the weight pass), up to 512 for the
// dense decode (the weight pass loops over 64 splits at a time).
constexpr int kMaxSplit = 64;
constexpr int kMaxSplitDense = 512;
constexpr int kCombOut = 64;                 // outputs per combine workgroup
constexpr int kCombGroups = kAttnThreads / (kCombOut / 4);   // 16 split groups

template <int MAXS>
__global__ __launch_bounds__(kAttnThreads) void sd_combine_kernel(const float* __restrict__ part, int nsplit, int Bh,
                                                                 int G, int Hq, int Hkv, uint16_t* __restrict__ out) {
    static_assert(MAXS % kWave == 0 && MAXS % kCombGroups == 0, "combine split layout");
    constexpr int kMaxSplit = MAXS;
    __shared__ float wgt[kMaxSplit];
    __shared__ float4 red[kCombGroups][kCombOut / 4];
    const int j = blockIdx.y, b = blockIdx.z, bj = b * Hkv + j;
    const int o0 = blockIdx.x * kCombOut;                  // first output, in [0, G*128)
    const int h = o0 / kHeadDim;
    const int q = threadIdx.x % (kCombOut / 4), sg = threadIdx.x / (kCombOut / 4);
    const int64_t row = int64_t(G) * kHeadDim;             // floats per split
    const float* pa = part + int64_t(bj) * nsplit * row + o0 + 4 * q;
    const float* pml = part + int64_t(Bh) * G * kHeadDim * nsplit + int64_t(bj) * nsplit * G * 2 + h * 2;
    float4 v[kMaxSplit / kCombGroups];
#pragma unroll
    for (int i = 0; i < kMaxSplit / kCombGroups; ++i) {
        const int s = sg + kCombGroups * i;
        v[i] = s < nsplit ? *reinterpret_cast<const float4*>(pa + s * row) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if (threadIdx.x < kWave) {
        const int lane = threadIdx.x;
        constexpr int kW = kMaxSplit / kWave;    // splits per lane
        float m[kW], l[kW];
        float M = -INFINITY;
#pragma unroll
        for (int i = 0; i < kW; ++i) {
            const int s = lane + kWave * i;
            m[i] = s < nsplit ? pml[s * G * 2] : -INFINITY;
            l[i] = s < nsplit ? pml[s * G * 2 + 1] : 0.f;
            M = fmaxf(M, m[i]);
        }
        M = wave_max_f(M);
        float f[kW], Lp = 0.f;
#pragma unroll
        for (int i = 0; i < kW; ++i) {
            f[i] = rescale(m[i], M);
            Lp = fmaf(l[i], f[i], Lp);
        }
        const float Lt = wave_sum_f(Lp);
#pragma unroll
        for (int i = 0; i < kW; ++i) {
            const int s = lane + kWave * i;
            wgt[s] = (s < nsplit && Lt > 0.f) ? f[i] / Lt : 0.f;
        }
    }
    __syncthreads();
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int i = 0; i < kMaxSplit / kCombGroups; ++i) {
        const int s = sg + kCombGroups * i;
        const float w = s < nsplit ? wgt[s] : 0.f;
        a.x = fmaf(v[i].x, w, a.x);
        a.y = fmaf(v[i].y, w, a.y);
        a.z = fmaf(v[i].z, w, a.z);
        a.w = fmaf(v[i].w, w, a.w);
    }
    red[sg][q] = a;
    __syncthreads();
    if (threadIdx.x < kCombOut / 4) {
        float4 t = red[0][threadIdx.x];
#pragma unroll
        for (int g = 1; g < kCombGroups; ++g) {
            const float4 u = red[g][threadIdx.x];
            t.x += u.x;
            t.y += u.y;
            t.z += u.z;
            t.w += u.w;
        }
        const int dd = (o0 % kHeadDim) + 4 * threadIdx.x;
        uint16_t* o = out + (int64_t(b) * Hq + j * G + h) * kHeadDim + dd;
        const uint32_t lo = uint32_t(f32_to_bf16_rne(t.x)) | (uint32_t(f32_to_bf16_rne(t.y)) << 16);
        const uint32_t hi = uint32_t(f32_to_bf16_rne(t.z)) | (uint32_t(f32_to_bf16_rne(t.w)) << 16);
        *reinterpret_cast<uint2*>(o) = make_uint2(lo, hi);
    }
}

template <int G>
static void launch_g(const AttendParams& p, dim3 grid, bool hostv, bool fuse, bool given, bool wide, size_t lds,
                     hipStream_t s, Timing t) {
    const dim3 block(kAttnThreads);
    // a fused Q select is the 4-wide one (Q.ncand <= 512 when fused)
    const int sq = select_width(p.last.ncand), sp = fuse ? select_width(p.P.ncand) : 0;
    constexpr int W = kDecodeWideSplits;
    if (wide && !hostv && !fuse) {
        // many pipelines (the unfused plan, or reused stages)
        if (given) launch(sd_flash_decode_kernel<G, false, kGiven, 0, W>, grid, block, lds, s, t, p);
        else if (sq == 4) launch(sd_flash_decode_kernel<G, false, 4, 0, W>, grid, block, lds, s, t, p);
        else if (sq == 16) launch(sd_flash_decode_kernel<G, false, 16, 0, W>, grid, block, lds, s, t, p);
        else launch(sd_flash_decode_kernel<G, false, kSelLds, 0, W>, grid, block, lds, s, t, p);
        return;
    }
    if (hostv) launch(sd_flash_decode_kernel<G, true, 4, 0>, grid, block, 0, s, t, p);
    else if (given) launch(sd_flash_decode_kernel<G, false, kGiven, 0>, grid, block, lds, s, t, p);
    else if (fuse && sp == 4) launch(sd_flash_decode_kernel<G, false, 4, 4>, grid, block, lds, s, t, p);
    else if (fuse && sp == 16) launch(sd_flash_decode_kernel<G, false, 4, 16>, grid, block, lds, s, t, p);
    else if (fuse) launch(sd_flash_decode_kernel<G, false, 4, kSelLds>, grid, block, lds, s, t, p);
    else if (sq == 4) launch(sd_flash_decode_kernel<G, false, 4, 0>, grid, block, lds, s, t, p);
    else if (sq == 16) launch(sd_flash_decode_kernel<G, false, 16, 0>, grid, block, lds, s, t, p);
    else launch(sd_flash_decode_kernel<G, false, kSelLds, 0>, grid, block, lds, s, t, p);
}

hipError_t launch_attend(sd_ctx* c, bool given, bool fused, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                         const int32_t* lengths, int32_t* kept, uint16_t* out, hipStream_t s, Timing t) {
    AttendParams p{};
    p.q = q;
    p.k = k;
    p.v = v;
    p.vpool = c->vc.pool;
    p.blk_slot = c->vc.blk_slot;
    p.vslots = c->vc.slots;
    p.vcopied = c->vfetch == SD_VALUE_FETCH_COPY;
    p.lengths = lengths;
    p.blocks = c->blocks;
    p.nblocks = c->nblocks;
    p.max_blocks = c->max_blocks;
    p.part = c->part;
    p.nsplit = c->nsplit;
    p.nsplit_a = c->nsplit_a;
    p.Bh = c->cfg.batch * c->cfg.num_kv_heads;
    p.tick = c->tick;
    const int S = c->S;
    p.last = stage_dev(c, S - 1);
    p.first_stage = S == 1;
    p.pp_koff = S >= 2 ? c->st[S - 2].koff : 0;
    p.last_scores = c->scores[S - 1];
    p.kept = kept;
    p.keep_total = c->keep_total;
    p.flag = c->flag;
    p.sink = c->cfg.sink;
    p.window = c->cfg.window;
    const bool fuse = fused && !given;
    if (fuse) {
        p.P = stage_dev(c, S - 2);
        p.p_first = S == 2;
        p.pp_koff_p = S >= 3 ? c->st[S - 3].koff : 0;
        p.p_scores = c->scores[S - 2];
        p.pre = c->pre;
        p.fuse_rq = c->fuse_rq;
    }
    const size_t lds = size_t(fuse ? fused_lds_words(p.P, p.p_first != 0, p.last, p.fuse_rq)
                                   : kept_lds_words(p.last, p.first_stage != 0)) * 4;
    p.Lmax = c->Lmax;
    p.Hq = c->cfg.num_q_heads;
    p.Hkv = c->cfg.num_kv_heads;
    p.scale_log2 = c->scale_log2;
    p.out = out;
    p.rec = c->rec;
    const dim3 grid(unsigned(pipe_grid(c->nsplit, p.Bh)));
    const bool hostv = c->cfg.values_on_host != 0;
    switch (c->G) {
        case 1: launch_g<1>(p, grid, hostv, fuse, given, c->decode_wide != 0, lds, s, t); break;
        case 2: launch_g<2>(p, grid, hostv, fuse, given, c->decode_wide != 0, lds, s, t); break;
        default: launch_g<4>(p, grid, hostv, fuse, given, c->decode_wide != 0, lds, s, t); break;
    }
    return hipGetLastError();
}

}  // namespace sd

namespace sd {

hipError_t launch_combine(sd_ctx* c, int nsplit, uint16_t* out, hipStream_t s, Timing t) {
    const int G = c->G;
    dim3 grid(G * kHeadDim / kCombOut, c->cfg.num_kv_heads, c->cfg.batch), block(kAttnThreads);
    static_assert(kAttnThreads % (kCombOut / 4) == 0 && kMaxSplitDense % kCombGroups == 0, "combine thread layout");
    static_assert(kHeadDim % kCombOut == 0, "a combine workgroup stays within one head");
    const int Bh = c->cfg.batch * c->cfg.num_kv_heads;
    const float* part = c->part;
    if (nsplit <= kMaxSplit)
        launch(sd_combine_kernel<kMaxSplit>, grid, block, 0, s, t, part, nsplit, Bh, G, c->cfg.num_q_heads,
               c->cfg.num_kv_heads, out);
    else
        launch(sd_combine_kernel<kMaxSplitDense>, grid, block, 0, s, t, part, nsplit, Bh, G, c->cfg.num_q_heads,
               c->cfg.num_kv_heads, out);
    return hipGetLastError();
}

hipError_t launch_dense(sd_ctx* c, const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* lengths,
                        hipStream_t s, Timing t) {
    AttendParams p{};
    p.q = q;
    p.k = k;
    p.v = v;
    p.lengths = lengths;
    p.flag = c->flag;
    p.part = c->part;
    p.nsplit = c->nsplit_d;
    p.Bh = c->cfg.batch * c->cfg.num_kv_heads;
    p.Lmax = c->Lmax;
    p.Hq = c->cfg.num_q_heads;
    p.Hkv = c->cfg.num_kv_heads;
    p.scale_log2 = c->scale_log2;
    const dim3 grid(c->nsplit_d, c->cfg.num_kv_heads, c->cfg.batch), block(kAttnThreads);
    switch (c->G) {
        case 1: launch(sd_dense_decode_kernel<1>, grid, block, 0, s, t, p); break;
        case 2: launch(sd_dense_decode_kernel<2>, grid, block, 0, s, t, p); break;
        default: launch(sd_dense_decode_kernel<4>, grid, block, 0, s, t, p); break;
    }
    return hipGetLastError();
}

}  // namespace sd

SD_PHASE_SETUP(attend)
