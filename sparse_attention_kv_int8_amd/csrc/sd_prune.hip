// Stacked pruning stages over the int8 key cache.
//
// Source: news article on InfiniteHiP ("韩国通过卸载键值缓存节约英伟达GPU内存，
// 实现18.95倍解码加速"), section "实现 7.24 倍的端到端解码加速": each pruning
// module cuts its input into fixed-length chunks, finds an approximate top
// token per chunk in parallel and passes only the K best chunks on; stacking
// modules refines a block-sparse mask.  The representative score of a chunk
// here is the maximum, over its tokens t = x, x + r, x + 2r, ... (t < L), of
// the exact integer score S_t = Q_j . K8_t, where Q_j is the sum of the int8
// query vectors of KV head j's query heads (global approximate scoring on
// quantised keys: HCAttention summary page, sections 摘要 and HCAttention).
//
// One kernel per stage.  The kernel of stage s > 0 first recomputes, in
// every workgroup, the kept set of stage s-1 from its scores (sd_select.h);
// workgroup 0 publishes it in kept_idx.  When stage s-1 is reused from an
// earlier step (the same article, same section: the modular design gives
// fine-grained control over caching the pruning stages), that kept set is
// read from kept_idx instead.  Then each workgroup scores its slice of stage
// s's candidates (the children of that kept set).  The kept set of the last
// stage (fused: of the last two) is selected by the attention kernel.

#include "sd_device.h"
#include "sd_internal.h"
#include "sd_select.h"

namespace sd {

constexpr int kPruneThreads = 256;
constexpr int kPruneWaves = kPruneThreads / kWave;
// PARTS staging: a wave's row scores, cpw x nrows <= kStageRows words (128
// for every geometry the plan admits: cpw x nrows = 8 per load slot x 8
// slots per batch x at most 2 batches), then one spare word per lane
constexpr int kStageRows = 256;
constexpr int kStageRowsPerWave = kStageRows + kWave;
// (kMaxCandPerWave, candidates per wave at most: sd_internal.h)

struct PruneParams {
    const uint16_t* q;        // [B][Hq][d]
    const int8_t* k8;         // [B][Hkv][Lmax][d]
    const int32_t* lengths;   // [B]
    int64_t Lmax;
    int Hq, Hkv, G, BH;
    int W;                    // workgroups per (request, KV head)
    int32_t* qgroup;          // [B][Hkv][d]
    int32_t* kept;            // [B][Hkv][keep_total]
    int keep_total;
    int32_t* flag;
    int stage;                // this kernel scores stage `stage`
    StageDev cur, prev;       // prev: the stage whose kept set is selected first (stage > 0)
    int cpw;                  // candidates per wave
    const int32_t* prev_scores;   // [B][Hkv][prev.ncand]
    int pp_koff;                  // kept_idx offset of stage - 2 (the previous stage's parents)
    int32_t* scores;              // [B][Hkv][cur.ncand]
    int nrows, rstride;           // key rows read per candidate, and their token stride
    int fuse_rq, fuse_m;          // fused next stage: children per chunk, stride ratio
    int32_t* pre;                 // fused next stage: [B][Hkv][cur.ncand * fuse_rq] children's scores
    const uint8_t* k4;            // first stage from the int4 sketch: [B][Hkv][k4_rows][64]
    int64_t k4_rows;
    // rows shared with the stage before the last (unfused plan, that stage's
    // stride twice the last's): children per chunk of the stage before, the
    // children's maxima over the rows that stage read ([B][Hkv][its ncand *
    // half_rq]), and, in the last stage's launch, the token offset of the
    // first row it reads itself (its stride)
    int half_rq;
    int32_t* parts;
    int odd_off;
};

// One load batch of a wave: CB candidates (starts xs, -1 = none) x NS8
// slots of 8 rows (8 lanes x 16 bytes per 128-byte int8 row).  load()
// issues every row load of the batch; score() consumes them, so the two
// can be separated by work that does not touch the rows (the first stage
// issues its loads before it forms the query).
template <int NS8, bool FUSE, bool PARTS = false>
struct RowBatch {
    static constexpr int CB = NS8 >= 8 ? 1 : 8 / NS8;     // candidates per batch
    static constexpr int NL = CB * NS8;                    // loads per batch
    u32x4 v[NL];
    bool ok[NL];

    __device__ __forceinline__ void load(const PruneParams& p, const int64_t (&xs)[CB], int64_t L,
                                         const int8_t* __restrict__ k8_bj) {
        const int lane = threadIdx.x & 63, row8 = lane >> 3, sl = lane & 7;
#pragma unroll
        for (int u = 0; u < NL; ++u) {
            const int c = u / NS8, it = u % NS8;
            const int i = it * 8 + row8;
            const int64_t t = xs[c] + int64_t(i) * p.rstride;
            ok[u] = xs[c] >= 0 && i < p.nrows && t < L;
            // every load issued, rows that do not count read as row 0 (in bounds) and masked by ok in
            // score(): a load under a branch makes the compiler wait for it before the next one
            const int64_t tc = ok[u] ? t : 0;
            v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(k8_bj + tc * kHeadDim) + sl);
        }
    }

    // Scores candidates first + c (c < CB, first + c < ncand, c < nvalid)
    // into out (and, with FUSE, every child's score into pre_bj; with PARTS,
    // every row's score into pre_bj, the batch's LDS staging rows, the other
    // lanes' stores going to spare[lane], the wave's 64 spare words).
    __device__ __forceinline__ void score(const PruneParams& p, const u32x4& qh, const u32x4& ql, int first,
                                          int nvalid, int32_t* __restrict__ out, int32_t* __restrict__ pre_bj,
                                          int* spare = nullptr) const {
        const StageDev& st = p.cur;
        const int lane = threadIdx.x & 63, row8 = lane >> 3;
        bool own[NS8];                             // row of slot it is one of this stage's samples
#pragma unroll
        for (int it = 0; it < NS8; ++it) own[it] = !FUSE || ((it * 8 + row8) % p.fuse_m) == 0;
        int best[CB];
#pragma unroll
        for (int c = 0; c < CB; ++c) best[c] = INT32_MIN;
#pragma unroll
        for (int u = 0; u < NL; ++u) {
            const u32x4 x = v[u];
            int ah = __builtin_amdgcn_sdot4((int)qh.x, (int)x.x, 0, false);
            ah = __builtin_amdgcn_sdot4((int)qh.y, (int)x.y, ah, false);
            ah = __builtin_amdgcn_sdot4((int)qh.z, (int)x.z, ah, false);
            ah = __builtin_amdgcn_sdot4((int)qh.w, (int)x.w, ah, false);
            int al = __builtin_amdgcn_sdot4((int)ql.x, (int)x.x, 0, false);
            al = __builtin_amdgcn_sdot4((int)ql.y, (int)x.y, al, false);
            al = __builtin_amdgcn_sdot4((int)ql.z, (int)x.z, al, false);
            al = __builtin_amdgcn_sdot4((int)ql.w, (int)x.w, al, false);
            const int s = sum8_i(ah * 64 + al);
            if (ok[u] && own[u % NS8]) best[u / NS8] = max(best[u / NS8], s);
            if (FUSE) {
                const int c = u / NS8, it = u % NS8;
                const int sub = max_groups_i(ok[u] ? s : INT32_MIN);
                if (lane == 0 && it < p.fuse_rq && c < nvalid && first + c < st.ncand)
                    pre_bj[int64_t(first + c) * p.fuse_rq + it] = sub;
            }
            if (PARTS) {
                // every row's score (INT32_MIN for rows that do not count),
                // one lane per row, into this batch's [candidate][row] rows
                // of the wave's LDS staging (pre_bj here; LDS writes leave
                // the load counter alone); store_child_max reduces them
                // (every lane stores, without a branch: the group's first
                // lane to its row, the others to a spare word of their own
                // past the rows; a branch here made the compiler wait for all
                // of the batch's loads at once)
                const int c = u / NS8, it = u % NS8;
                int* at = (lane & 7) == 0 ? pre_bj + c * p.nrows + it * 8 + row8 : spare + lane;
                *at = ok[u] ? s : INT32_MIN;
            }
        }
#pragma unroll
        for (int c = 0; c < CB; ++c) {
            const int m = max_groups_i(best[c]);
            if (lane == 0 && c < nvalid && first + c < st.ncand) out[first + c] = m;
        }
    }
};

// PARTS: the wave's staged row scores ([cpw][nrows] in LDS, 4 rows per
// child of the next stage) reduced to each child's maximum and stored
// [candidate][child] from candidate `first` on: one store for the wave,
// whole cache lines when cpw * half_rq is a multiple of 32.
__device__ __forceinline__ void store_child_max(const PruneParams& p, const int* rows, int first, int cpw,
                                                int32_t* __restrict__ parts_bj) {
    const int lane = threadIdx.x & 63;
    const int rq = p.half_rq;
    for (int l = lane; l < cpw * rq; l += kWave) {
        const int c = l / rq, k = l - c * rq;
        const i32x4 r = *reinterpret_cast<const i32x4*>(rows + c * p.nrows + 4 * k);
        if (first + c < p.cur.ncand) parts_bj[int64_t(first) * rq + l] = max(max(r.x, r.y), max(r.z, r.w));
    }
}

// One load batch of the last stage's own rows when the stage before it
// read every other one (its stride twice the last's; 8 rows per last-stage
// chunk): rows x + odd_off + r rstride, r < 4, of 16 candidates, two per
// load slot (lanes [0, 32): candidate 2 u, lanes [32, 64): 2 u + 1; 8 lanes
// per 128-byte row).  A candidate's score is the larger of the maximum over
// these rows and the maximum over the other four (parts, stored by the
// stage before, which read them): the maximum over all eight, exactly, with
// half the rows read.
struct OddBatch {
    static constexpr int CB = 16;
    u32x4 v[8];
    bool ok[8];
    int part;          // lane c < CB: candidate c's stored maximum

    __device__ __forceinline__ void load(const PruneParams& p, const int* xs, const int* pidx, int64_t L,
                                         const int8_t* __restrict__ k8_bj, const int32_t* __restrict__ parts_bj) {
        const int lane = threadIdx.x & 63, r4 = (lane >> 3) & 3, hf = lane >> 5, sl = lane & 7;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int x = xs[2 * u + hf];
            const int64_t t = int64_t(x) + p.odd_off + int64_t(r4) * p.rstride;
            ok[u] = x >= 0 && t < L;
            const int64_t tc = ok[u] ? t : 0;      // issued for every lane (masked in score)
            v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(k8_bj + tc * kHeadDim) + sl);
        }
        const int pi = lane < CB ? pidx[lane] : -1;
        part = pi >= 0 ? parts_bj[pi] : INT32_MIN;
    }

    __device__ __forceinline__ void score(const PruneParams& p, const u32x4& qh, const u32x4& ql, int first,
                                          int nvalid, int32_t* __restrict__ out) const {
        const int lane = threadIdx.x & 63;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const u32x4 x = v[u];
            int ah = __builtin_amdgcn_sdot4((int)qh.x, (int)x.x, 0, false);
            ah = __builtin_amdgcn_sdot4((int)qh.y, (int)x.y, ah, false);
            ah = __builtin_amdgcn_sdot4((int)qh.z, (int)x.z, ah, false);
            ah = __builtin_amdgcn_sdot4((int)qh.w, (int)x.w, ah, false);
            int al = __builtin_amdgcn_sdot4((int)ql.x, (int)x.x, 0, false);
            al = __builtin_amdgcn_sdot4((int)ql.y, (int)x.y, al, false);
            al = __builtin_amdgcn_sdot4((int)ql.z, (int)x.z, al, false);
            al = __builtin_amdgcn_sdot4((int)ql.w, (int)x.w, al, false);
            int h = sum8_i(ah * 64 + al);
            h = ok[u] ? h : INT32_MIN;
            h = max(h, dpp_i<kDppRor8>(h));
            const int c0 = 2 * u, c1 = 2 * u + 1;
            const int m0 = max(max(__builtin_amdgcn_readlane(h, 0), __builtin_amdgcn_readlane(h, 16)),
                               __builtin_amdgcn_readlane(part, c0));
            const int m1 = max(max(__builtin_amdgcn_readlane(h, 32), __builtin_amdgcn_readlane(h, 48)),
                               __builtin_amdgcn_readlane(part, c1));
            if (lane == 0) {
                if (c0 < nvalid && first + c0 < p.cur.ncand) out[first + c0] = m0;
                if (c1 < nvalid && first + c1 < p.cur.ncand) out[first + c1] = m1;
            }
        }
    }
};

// One load batch of the first stage from the int4 sketch: 4 lanes x 16
// bytes per 64-byte sketch row (lane = 4 * row + part; part p holds
// channels [32 p, 32 p + 32)), 16 rows per load slot, NS16 slots per
// candidate, 8 loads per batch (CB = 8 / NS16 candidates).  Word m of a
// part holds channels 32 p + 8 m + k as two's-complement nibbles k = 0..7,
// which v_dot8_i32_i4 multiplies pairwise with the same nibbles of a query
// digit word (split_query4d); S = d0 . K4 + 16 (d1 . K4) + 256 (d2 . K4),
// exact in int32.  Every first-stage sample t is a multiple of the stride,
// at sketch row t / stride.
template <int NS16>
struct SketchBatch {
    static constexpr int CB = 8 / NS16;
    static constexpr int NL = CB * NS16;
    u32x4 v[NL];
    bool ok[NL];

    __device__ __forceinline__ void load(const PruneParams& p, const int64_t (&xs)[CB], int64_t L,
                                         const uint8_t* __restrict__ k4_bj) {
        const int lane = threadIdx.x & 63, r16 = lane >> 2, part = lane & 3;
#pragma unroll
        for (int u = 0; u < NL; ++u) {
            const int c = u / NS16, it = u % NS16;
            const int i = it * 16 + r16;
            const int64_t t = xs[c] + int64_t(i) * p.rstride;
            ok[u] = xs[c] >= 0 && i < p.nrows && t < L;
            const int64_t row = ok[u] ? int64_t(int(xs[c]) / p.rstride) + i : 0;   // = t / rstride (row 0: masked)
            v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(k4_bj + row * (kHeadDim / 2)) + part);
        }
    }

    __device__ __forceinline__ void score(const PruneParams& p, const uint32_t (&d0)[4], const uint32_t (&d1)[4],
                                          const uint32_t (&d2)[4], int first, int nvalid,
                                          int32_t* __restrict__ out) const {
        const int lane = threadIdx.x & 63;
        int best[CB];
#pragma unroll
        for (int c = 0; c < CB; ++c) best[c] = INT32_MIN;
#pragma unroll
        for (int u = 0; u < NL; ++u) {
            const int w[4] = {int(v[u].x), int(v[u].y), int(v[u].z), int(v[u].w)};
            int a0 = 0, a1 = 0, a2 = 0;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                a0 = __builtin_amdgcn_sdot8(int(d0[m]), w[m], a0, false);
                a1 = __builtin_amdgcn_sdot8(int(d1[m]), w[m], a1, false);
                a2 = __builtin_amdgcn_sdot8(int(d2[m]), w[m], a2, false);
            }
            int sv = a0 + 16 * a1 + 256 * a2;
            sv += dpp_i<kDppXor1>(sv);
            sv += dpp_i<kDppXor2>(sv);                 // the row's score in its 4 lanes
            if (ok[u]) best[u / NS16] = max(best[u / NS16], sv);
        }
#pragma unroll
        for (int c = 0; c < CB; ++c) {
            // max over the 16 row groups: groups of a row of 16 lanes, then the four rows
            int m = best[c];
            m = max(m, dpp_i<0x124>(m));               // row_ror:4
            m = max(m, dpp_i<kDppRor8>(m));
            m = max(max(__builtin_amdgcn_readlane(m, 0), __builtin_amdgcn_readlane(m, 16)),
                    max(__builtin_amdgcn_readlane(m, 32), __builtin_amdgcn_readlane(m, 48)));
            if (lane == 0 && c < nvalid && first + c < p.cur.ncand) out[first + c] = m;
        }
    }
};

// Score `cpw` candidates per wave.  NS8 = rows per candidate / 8 (rounded up);
// each load slot covers 8 rows (8 lanes x 16 bytes per 128-byte row).
// cstart: LDS, the starts of this wave's candidates (-1 = none).  Rows
// t = x + i * rstride, i < nrows, are read (8 lanes per row, 8 rows per load
// slot).  Without FUSE they are this stage's samples.  With FUSE they are
// the next stage's samples (rstride = its stride, one 8-row slot per child
// chunk): this stage's score is the max over rows i % fuse_m == 0 (its own
// samples), and each slot's max is written as that child's score.
template <int NS8, bool FUSE, bool PARTS = false>
__device__ __forceinline__ void score_slice(const PruneParams& p, const int* cstart, int64_t L,
                                            const int8_t* __restrict__ k8_bj, const u32x4& qh, const u32x4& ql,
                                            int first, int32_t* __restrict__ out, int32_t* __restrict__ pre_bj,
                                            int* stage_rows = nullptr) {
    using RB = RowBatch<NS8, FUSE, PARTS>;
    for (int c0 = 0; c0 < p.cpw; c0 += RB::CB) {
        int64_t xs[RB::CB];
#pragma unroll
        for (int c = 0; c < RB::CB; ++c) xs[c] = (c0 + c < p.cpw) ? cstart[c0 + c] : -1;
        RB rb;
        rb.load(p, xs, L, k8_bj);
        rb.score(p, qh, ql, first + c0, p.cpw - c0, out, PARTS ? stage_rows + c0 * p.nrows : pre_bj,
                 PARTS ? stage_rows + kStageRows : nullptr);
    }
    if (PARTS) store_child_max(p, stage_rows, first, p.cpw, pre_bj);
}

// hi/lo int8 split of the 16 query dims [16 sl, 16 sl + 16): Q = 64 hi + lo,
// lo in [-32, 31], so both halves fit int8 and S = 64 (hi . k) + (lo . k).
__device__ __forceinline__ void split_query(const int* Qlds, int sl, u32x4& qh, u32x4& ql) {
    uint32_t h4[4], l4[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        uint32_t hw = 0, lw = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int Q = Qlds[sl * 16 + w * 4 + u];
            const int lo = ((Q + 32) & 63) - 32;
            const int hi = (Q - lo) >> 6;
            hw |= (uint32_t(hi) & 0xffu) << (8 * u);
            lw |= (uint32_t(lo) & 0xffu) << (8 * u);
        }
        h4[w] = hw;
        l4[w] = lw;
    }
    qh = u32x4{h4[0], h4[1], h4[2], h4[3]};
    ql = u32x4{l4[0], l4[1], l4[2], l4[3]};
}

// Query digit words for SketchBatch: Q = d0 + 16 d1 + 256 d2 with every
// digit in [-8, 7] (balanced base 16; |Q| <= 508 < 7 (1 + 16 + 256)), and
// word m of digit i holds d_i of channels 32 part + 8 m + k as
// two's-complement nibbles k = 0..7.
__device__ __forceinline__ void split_query4d(const int* Qlds, int part, uint32_t (&d0)[4], uint32_t (&d1)[4],
                                              uint32_t (&d2)[4]) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        uint32_t w0 = 0, w1 = 0, w2 = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            int Q = Qlds[32 * part + 8 * m + k];
            const int e0 = ((Q + 8) & 15) - 8;
            Q = (Q - e0) >> 4;
            const int e1 = ((Q + 8) & 15) - 8;
            const int e2 = (Q - e1) >> 4;
            w0 |= (uint32_t(e0) & 0xfu) << (4 * k);
            w1 |= (uint32_t(e1) & 0xfu) << (4 * k);
            w2 |= (uint32_t(e2) & 0xfu) << (4 * k);
        }
        d0[m] = w0;
        d1[m] = w1;
        d2[m] = w2;
    }
}

// Stages other than the first unfused one: the previous stage's kept set
// (selected here, or given), then this workgroup's slice of the candidates.
// Lraw: the request's length as loaded (sanitised here, where first needed,
// so that the head select's loads do not wait for it).
// HR (rows shared with the stage before the last): 1, this stage is the
// one before the last and also stores its children's maxima (parts); 2,
// this is the last stage and reads only its rows that the stage before did
// not (OddBatch; 16 candidates per wave).
template <int NS8, int SEL, bool FUSE, int HR>
__device__ __forceinline__ void score_later(const PruneParams& p, int bj, int wgi, int b, int j, int32_t Lraw,
                                            int32_t* kept_bj, const int8_t* __restrict__ k8_bj,
                                            int32_t* scores_bj, uint32_t* dyn, int* Qlds, unsigned* tmp,
                                            int* cstart, int* cpre, int* stage_rows) {
    static_assert(HR != 2 || (SEL != 0 && SEL != kGiven && !FUSE), "odd rows: the stage before ran this step");
    const int wave = threadIdx.x >> 6;
    const int sl = threadIdx.x & 7;
    const int32_t* parents = nullptr;
    int64_t L = 0;
    if constexpr (SEL == 0 || SEL == kGiven) {
        const bool bad = Lraw < 1 || Lraw > p.Lmax;
        L = bad ? 0 : Lraw;
        // the first stage this step runs: flags a bad length and forms the
        // group query codes, which the later stages read
        if (bad && wgi == 0 && threadIdx.x == 0) atomicOr(p.flag, 1);
        group_query_codes(p.q + int64_t(b) * p.Hq * kHeadDim, j, p.G, Qlds, nullptr);
        if (wgi == 0 && threadIdx.x < kHeadDim)
            p.qgroup[int64_t(bj) * kHeadDim + threadIdx.x] = Qlds[threadIdx.x];
    }
    if constexpr (SEL == kGiven) {
        // the previous stage is reused: its kept set is read from kept_idx
        int* sel = reinterpret_cast<int*>(dyn + p.prev.ncand);
        given_kept<kPruneThreads>(p.prev, kept_bj + p.prev.koff, L, sel, tmp);
        parents = sel;
    } else if constexpr (SEL != 0) {
        // the group query load is issued together with the previous scores' loads
        const int qval = threadIdx.x < kHeadDim ? p.qgroup[int64_t(bj) * kHeadDim + threadIdx.x] : 0;
        // kept set of the previous stage (its own parents are in kept_idx
        // already).  The length bound is Lmax here: a selected candidate has
        // a score, so it starts below the length anyway.
        int* sel = reinterpret_cast<int*>(dyn + p.prev.ncand);
        const int32_t* pp = p.stage >= 2 ? kept_bj + p.pp_koff : nullptr;
        // HR = 2: the kept chunks' indices too (after the select's words)
        int* pidx = HR == 2 ? reinterpret_cast<int*>(dyn + kept_lds_words(p.prev, p.stage == 1)) : nullptr;
        const int nk = kept_of_stage<kPruneThreads, SEL>(p.prev, p.stage == 1, p.prev_scores + int64_t(bj) * p.prev.ncand,
                                                         pp, p.Lmax, dyn, tmp, p.stage, pidx);
        if (HR == 2)
            for (int i = nk + threadIdx.x; i < p.prev.keep; i += kPruneThreads) pidx[i] = -1;
        L = length_here(Lraw, p.Lmax);
        for (int i = nk + threadIdx.x; i < p.prev.keep; i += kPruneThreads) sel[i] = -1;
        if (threadIdx.x < kHeadDim) Qlds[threadIdx.x] = qval;
        __syncthreads();
        parents = sel;
    }
    SD_PHASE(p.stage, 1);
    // the starts of this workgroup's candidates, one thread each
    const int wg_first = wgi * kPruneWaves * p.cpw;
    if (int(threadIdx.x) < kPruneWaves * p.cpw) {
        const int ci = wg_first + threadIdx.x;
        const int x = int(cand_start(p.cur, SEL == 0, parents, ci, L));
        cstart[threadIdx.x] = x;
        if constexpr (HR == 2) {
            // this candidate's stored maximum: it is child ci % rq of kept
            // chunk ci / rq of the stage before (index pidx there)
            const int* pidx = reinterpret_cast<const int*>(dyn + kept_lds_words(p.prev, p.stage == 1));
            cpre[threadIdx.x] = x >= 0 ? pidx[ci / p.half_rq] * p.half_rq + ci % p.half_rq : -1;
        }
    }
    u32x4 qh, ql;
    split_query(Qlds, sl, qh, ql);
    __syncthreads();

    const int first = wg_first + wave * p.cpw;
    if constexpr (HR == 2) {
        OddBatch ob;
        ob.load(p, cstart + wave * p.cpw, cpre + wave * p.cpw, L, k8_bj,
                p.parts + int64_t(bj) * p.prev.ncand * p.half_rq);
        ob.score(p, qh, ql, first, p.cpw, scores_bj);
    } else {
        score_slice<NS8, FUSE, HR == 1>(p, cstart + wave * p.cpw, L, k8_bj, qh, ql, first, scores_bj,
                                        FUSE     ? p.pre + int64_t(bj) * p.cur.ncand * p.fuse_rq
                                        : HR == 1 ? p.parts + int64_t(bj) * p.cur.ncand * p.half_rq
                                                  : nullptr,
                                        HR == 1 ? stage_rows + wave * kStageRowsPerWave : nullptr);
    }
    if constexpr (SEL != 0 && SEL != kGiven) {
        // workgroup 0 publishes the previous stage's kept set (ascending,
        // -1 padded); stored last, so no barrier waits on these stores
        if (wgi == 0)
            for (int i = threadIdx.x; i < p.prev.keep; i += kPruneThreads) kept_bj[p.prev.koff + i] = parents[i];
    }
}

// One instantiation per (rows per candidate / 8, select code of the
// previous stage (0 = stage 0, kGiven = the previous stage reused), fused
// next stage, int4 sketch): each launch carries only its own path, which
// keeps code size and scalar-register pressure down.
template <int NS8, int SEL, bool FUSE, bool Q4 = false, int HR = 0>
__global__ __launch_bounds__(kPruneThreads) void sd_prune_stage_kernel(PruneParams p) {
    static_assert(!Q4 || (SEL == 0 && !FUSE && HR == 0), "the int4 sketch serves the unfused first stage only");
    static_assert(HR == 0 || !FUSE, "rows shared with the stage before: unfused plan");
    extern __shared__ uint32_t dyn[];      // the previous stage's select (kept_lds_words)
    __shared__ int Qlds[kHeadDim];
    __shared__ unsigned tmp[32];
    __shared__ int cstart[kPruneWaves * kMaxCandPerWave];
    __shared__ int cpre[HR == 2 ? kPruneWaves * OddBatch::CB : 1];   // HR = 2: stored-maximum indices
    __shared__ __align__(16) int stage_rows[HR == 1 ? kPruneWaves * kStageRowsPerWave : 1];   // HR = 1: row scores

    SD_PHASE(p.stage, 0);
    // all workgroups of a (request, KV head) on one XCD (sd_device.h): the
    // scores they write stay in that XCD's L2 for the kernel after
    const PipeSlot ps = pipe_slot(p.W, p.BH);
    if (ps.bj < 0) return;
    const int bj = ps.bj, wgi = ps.w;
    const int b = bj / p.Hkv, j = bj - b * p.Hkv;
    // the length is sanitised where each path first needs it (an invalid
    // request has no candidates)
    const int32_t Lraw = load_length(p.lengths, b);
    // the first stage's query pair, loaded together with the length
    const uint32_t qpr = (Q4 || (SEL == 0 && !FUSE)) ? query_pair(p.q + int64_t(b) * p.Hq * kHeadDim, j, p.G) : 0u;
    int32_t* kept_bj = p.kept + int64_t(bj) * p.keep_total;

    const int8_t* k8_bj = p.k8 + int64_t(bj) * p.Lmax * kHeadDim;
    const uint8_t* k4_bj = Q4 ? p.k4 + int64_t(bj) * p.k4_rows * (kHeadDim / 2) : nullptr;
    int32_t* scores_bj = p.scores + int64_t(bj) * p.cur.ncand;
    const int wave = threadIdx.x >> 6;
    const int sl = threadIdx.x & 7;
    if constexpr (Q4) {
        // First stage from the int4 sketch, one load batch per wave (cpw =
        // CB): rows loaded first, query codes formed while they are in flight.
        constexpr int NS16 = NS8 >= 2 ? NS8 / 2 : 1;
        using SB = SketchBatch<NS16>;
        const bool bad = Lraw < 1 || Lraw > p.Lmax;
        const int64_t L = bad ? 0 : Lraw;
        const int first = (wgi * kPruneWaves + wave) * p.cpw;
        int64_t xs[SB::CB];
#pragma unroll
        for (int c = 0; c < SB::CB; ++c) xs[c] = c < p.cpw ? cand_start(p.cur, true, nullptr, first + c, L) : -1;
        SB sb;
        sb.load(p, xs, L, k4_bj);
        if (bad && wgi == 0 && threadIdx.x == 0) atomicOr(p.flag, 1);
        group_query_codes(qpr, j, p.G, Qlds, nullptr);
        if (wgi == 0 && threadIdx.x < kHeadDim)
            p.qgroup[int64_t(bj) * kHeadDim + threadIdx.x] = Qlds[threadIdx.x];
        uint32_t d0[4], d1[4], d2[4];
        split_query4d(Qlds, threadIdx.x & 3, d0, d1, d2);
        sb.score(p, d0, d1, d2, first, p.cpw, scores_bj);
    } else if constexpr (SEL == 0 && !FUSE) {
        // First stage, one load batch per wave (cpw = CB): the candidate
        // starts follow from the indices, so the rows are loaded first and
        // the query codes are formed while the loads are in flight.
        using RB = RowBatch<NS8, false, HR == 1>;
        const bool bad = Lraw < 1 || Lraw > p.Lmax;
        const int64_t L = bad ? 0 : Lraw;
        const int first = (wgi * kPruneWaves + wave) * p.cpw;
        int64_t xs[RB::CB];
#pragma unroll
        for (int c = 0; c < RB::CB; ++c) xs[c] = c < p.cpw ? cand_start(p.cur, true, nullptr, first + c, L) : -1;
        RB rb;
        rb.load(p, xs, L, k8_bj);
        if (bad && wgi == 0 && threadIdx.x == 0) atomicOr(p.flag, 1);
        group_query_codes(qpr, j, p.G, Qlds, nullptr);
        if (wgi == 0 && threadIdx.x < kHeadDim)
            p.qgroup[int64_t(bj) * kHeadDim + threadIdx.x] = Qlds[threadIdx.x];
        u32x4 qh, ql;
        split_query(Qlds, sl, qh, ql);
        int* rows_w = stage_rows + wave * kStageRowsPerWave;
        rb.score(p, qh, ql, first, p.cpw, scores_bj, HR == 1 ? rows_w : nullptr, HR == 1 ? rows_w + kStageRows : nullptr);
        if (HR == 1) store_child_max(p, rows_w, first, p.cpw, p.parts + int64_t(bj) * p.cur.ncand * p.half_rq);
    } else {
        score_later<NS8, SEL, FUSE, HR>(p, bj, wgi, b, j, Lraw, kept_bj, k8_bj, scores_bj, dyn, Qlds, tmp, cstart,
                                        cpre, stage_rows);
    }
    SD_PHASE(p.stage, 2);
}

StageDev stage_dev(const sd_ctx* c, int st) {
    const StageGeom& g = c->st[st];
    StageDev d;
    d.chunk = g.chunk;
    d.stride = g.stride;
    d.keep = g.keep;
    d.nsamp = g.nsamp;
    d.ncand = g.ncand;
    d.koff = g.koff;
    d.ratio = st ? c->st[st - 1].chunk / g.chunk : 1;
    return d;
}

hipError_t launch_prune_stage(sd_ctx* c, int st, bool given, bool fused, const uint16_t* q, const int8_t* k8,
                              const uint8_t* k4, const int32_t* lengths, int32_t* kept, hipStream_t s, Timing t) {
    PruneParams p{};
    p.q = q;
    p.k8 = k8;
    p.k4 = k4;
    p.k4_rows = c->sketch_rows;
    p.lengths = lengths;
    p.Lmax = c->Lmax;
    p.Hq = c->cfg.num_q_heads;
    p.Hkv = c->cfg.num_kv_heads;
    p.G = c->G;
    p.BH = c->cfg.batch * c->cfg.num_kv_heads;
    p.W = c->st[st].nwg;
    p.qgroup = c->qgroup;
    p.kept = kept;
    p.keep_total = c->keep_total;
    p.flag = c->flag;
    p.stage = st;
    p.cur = stage_dev(c, st);
    p.cpw = c->st[st].per_wg / kPruneWaves;
    p.scores = c->scores[st];
    p.nrows = c->st[st].nrows;
    p.rstride = c->st[st].rstride;
    const bool fuse = fused && st == c->S - 2;
    p.fuse_rq = fuse ? c->fuse_rq : 0;
    p.fuse_m = fuse ? c->fuse_m : 1;
    p.pre = fuse ? c->pre : nullptr;
    const bool q4 = k4 != nullptr && st == 0 && !fuse;
    // rows shared between the last two stages (unfused plan): stage S-2
    // stores its children's maxima, unless scored from the int4 sketch;
    // stage S-1 then reads only its other rows, when stage S-2 ran in this
    // step (not reused: `given`) and stored them
    const int hr = !c->half || fused                                         ? 0
                   : st == c->S - 2                                          ? (q4 ? 0 : 1)
                   : st == c->S - 1 && !given && !(st == 1 && k4 != nullptr) ? 2
                                                                             : 0;
    p.half_rq = hr ? c->half_rq : 0;
    p.parts = hr ? c->pre : nullptr;
    p.odd_off = 0;
    if (hr == 2) {
        p.nrows = 4;
        p.rstride = c->st[st - 1].stride;
        p.odd_off = c->st[st].stride;
        p.cpw = OddBatch::CB;
        p.W = (p.cur.ncand + kPruneWaves * p.cpw - 1) / (kPruneWaves * p.cpw);
    }
    size_t words = 0;
    if (st > 0) {
        p.prev = stage_dev(c, st - 1);
        p.prev_scores = c->scores[st - 1];
        p.pp_koff = st >= 2 ? c->st[st - 2].koff : 0;
        if (!given) words = size_t(kept_lds_words(p.prev, st == 1)) + (hr == 2 ? size_t(p.prev.keep) : 0);
        else words = size_t(p.prev.ncand + p.prev.keep + 1);
    }
    const size_t lds = words * 4;
    const int ns8 = (p.nrows + 7) >> 3;
    const int sel = st == 0 ? 0 : given ? kGiven : select_width(p.prev.ncand);
    if (q4) {
        // one batch of int4 candidates per wave (SketchBatch: 8 / NS16)
        const int ns8p = ns8 == 1 ? 1 : ns8 == 2 ? 2 : ns8 <= 4 ? 4 : 8;
        p.cpw = 8 / (ns8p >= 2 ? ns8p / 2 : 1);
        p.W = (p.cur.ncand + kPruneWaves * p.cpw - 1) / (kPruneWaves * p.cpw);
    }
    const dim3 grid(unsigned(pipe_grid(p.W, p.BH))), block(kPruneThreads);
#define SD_K(N, S, F, Q) launch(sd_prune_stage_kernel<N, S, F, Q>, grid, block, lds, s, t, p)
#define SD_KH(N, S, H) launch(sd_prune_stage_kernel<N, S, false, false, H>, grid, block, lds, s, t, p)
#define SD_NS(S)                                               \
    if (fuse) {                                                \
        if (ns8 <= 2) SD_K(2, S, true, false);                 \
        else if (ns8 <= 4) SD_K(4, S, true, false);            \
        else SD_K(8, S, true, false);                          \
    } else if (hr == 1) {                                      \
        if (ns8 == 1) SD_KH(1, S, 1);                          \
        else if (ns8 == 2) SD_KH(2, S, 1);                     \
        else if (ns8 <= 4) SD_KH(4, S, 1);                     \
        else SD_KH(8, S, 1);                                   \
    } else {                                                   \
        if (ns8 == 1) SD_K(1, S, false, false);                \
        else if (ns8 == 2) SD_K(2, S, false, false);           \
        else if (ns8 <= 4) SD_K(4, S, false, false);           \
        else SD_K(8, S, false, false);                         \
    }
    if (hr == 2) {
        // the stage before ran and was selected here: never kGiven
        if (sel == 4) SD_KH(1, 4, 2);
        else if (sel == 16) SD_KH(1, 16, 2);
        else SD_KH(1, kSelLds, 2);
    } else if (q4) {
        if (ns8 == 1) SD_K(1, 0, false, true);
        else if (ns8 == 2) SD_K(2, 0, false, true);
        else if (ns8 <= 4) SD_K(4, 0, false, true);
        else SD_K(8, 0, false, true);
    } else if (sel == 0) { SD_NS(0); }
    else if (sel == kGiven) { SD_NS(kGiven); }
    else if (sel == 4) { SD_NS(4); }
    else if (sel == 16) { SD_NS(16); }
    else { SD_NS(kSelLds); }
#undef SD_NS
#undef SD_KH
#undef SD_K
    return hipGetLastError();
}

}  // namespace sd

SD_PHASE_SETUP(prune)
