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
// Selection order is (score descending, chunk start ascending).
//
// One kernel per stage.  Workgroups score disjoint slices of the stage's
// candidates; the last workgroup to finish for a (request, KV head) runs an
// exact radix select over all candidate scores in LDS, writes the kept
// starts (ascending) and, after the last stage, the attended block list:
// kept chunks plus the sink and recent window (page "KV Cache 与长上下文推理",
// section "KV Cache 压缩技术", StreamingLLM).
#include "sd_device.h"
#include "sd_internal.h"

namespace sd {

constexpr int kPruneThreads = 256;
constexpr int kPruneWaves = kPruneThreads / kWave;

struct PruneParams {
    const uint16_t* q;        // [B][Hq][d]
    const int8_t* k8;         // [B][Hkv][Lmax][d]
    const int32_t* lengths;   // [B]
    int64_t Lmax;
    int Hq, Hkv, G;
    int32_t* qgroup;          // [B][Hkv][d]
    int32_t* kept;            // [B][Hkv][keep_total]
    int keep_total;
    int32_t* flag;
    // this stage
    int stage;
    int chunk, stride, keep, nsamp, ncand, koff, cpw;
    int prev_koff, ratio;     // stage > 0: parent list offset, children per parent
    int32_t* scores;          // [B][Hkv][ncand]
    unsigned* counter;        // [B][Hkv]
    int nwg;
    int last_stage;
    // attended set (last stage)
    uint32_t* blocks;         // [B][Hkv][max_blocks]
    int32_t* nblocks;         // [B][Hkv]
    int max_blocks;
    int sink, window;
};

// Start of candidate i (token position), or -1 if it does not exist.
__device__ __forceinline__ int64_t cand_start(const PruneParams& p, const int32_t* parents, int i,
                                              int64_t L) {
    if (i >= p.ncand) return -1;
    int64_t x;
    if (p.stage == 0) {
        x = int64_t(i) * p.chunk;
    } else {
        const int par = parents[i / p.ratio];
        if (par < 0) return -1;
        x = int64_t(par) + int64_t(i % p.ratio) * p.chunk;
    }
    return x < L ? x : -1;
}

// Exact top-K of n keys (0 = no candidate; otherwise larger is better, ties
// to the lower index).  keys: LDS [n].  Writes the kept indices ascending to
// sel[0..kept) and returns kept = min(K, #valid).
__device__ int select_top(const uint32_t* keys, int n, int K, int* sel, unsigned* hist, unsigned* tmp) {
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    // valid count, min and max key
    unsigned cnt = 0, kmn = 0xffffffffu, kmx = 0;
    for (int i = tid; i < n; i += kPruneThreads) {
        const unsigned k = keys[i];
        if (k) { ++cnt; kmn = min(kmn, k); kmx = max(kmx, k); }
    }
    for (int o = 32; o > 0; o >>= 1) cnt += (unsigned)__shfl_xor((int)cnt, o);
    kmn = wave_min_u(kmn);
    kmx = wave_max_u(kmx);
    // tmp[0..3] cnt, [4..7] min, [8..11] max per wave
    if (lane == 0) { tmp[wid] = cnt; tmp[4 + wid] = kmn; tmp[8 + wid] = kmx; }
    __syncthreads();
    unsigned nvalid = 0; kmn = 0xffffffffu; kmx = 0;
    for (int w = 0; w < kPruneWaves; ++w) { nvalid += tmp[w]; kmn = min(kmn, tmp[4 + w]); kmx = max(kmx, tmp[8 + w]); }
    __syncthreads();

    unsigned T = 0;          // threshold key
    int need_eq = 0;         // how many keys equal to T are kept (lowest indices)
    if (int(nvalid) > K) {
        const unsigned diff = kmx ^ kmn;
        int bits = diff ? 32 - __clz(diff) : 0;      // low bits that differ
        unsigned prefix = bits >= 32 ? 0u : (kmx >> bits) << bits;
        int remaining = K;
        while (bits > 0) {
            const int w = bits < 8 ? bits : 8;
            const int shift = bits - w;
            for (int i = tid; i < 256; i += kPruneThreads) hist[i] = 0;
            __syncthreads();
            const unsigned hi_mask = bits >= 32 ? 0u : ~((1u << bits) - 1u);
            for (int i = tid; i < n; i += kPruneThreads) {
                const unsigned k = keys[i];
                if (k && (k & hi_mask) == (prefix & hi_mask))
                    atomicAdd(hist + ((k >> shift) & ((1u << w) - 1u)), 1u);
            }
            __syncthreads();
            if (wid == 0) {
                // lane l owns bins 255-4l .. 252-4l (descending digit order)
                unsigned h[4], s = 0;
                for (int u = 0; u < 4; ++u) { h[u] = hist[255 - 4 * lane - u]; s += h[u]; }
                const unsigned incl = wave_incl_scan(s), excl = incl - s;
                if (excl < unsigned(remaining) && unsigned(remaining) <= incl) {
                    unsigned c = excl;
                    for (int u = 0; u < 4; ++u) {
                        if (c + h[u] >= unsigned(remaining)) {
                            tmp[12] = unsigned(255 - 4 * lane - u);
                            tmp[13] = c;
                            break;
                        }
                        c += h[u];
                    }
                }
            }
            __syncthreads();
            const unsigned dd = tmp[12], above = tmp[13];
            remaining -= int(above);
            prefix |= dd << shift;
            bits = shift;
            __syncthreads();
        }
        T = prefix;
        need_eq = remaining;
    }
    // Compaction in index order: thread t owns the contiguous range [i0, i1).
    const int per = (n + kPruneThreads - 1) / kPruneThreads;
    const int i0 = min(n, tid * per), i1 = min(n, i0 + per);
    unsigned g = 0, e = 0;
    for (int i = i0; i < i1; ++i) {
        const unsigned k = keys[i];
        g += k > T;
        e += (k == T) && k;
    }
    unsigned total;
    const unsigned ex = block_excl_scan<kPruneThreads>((g << 16) | e, tmp + 16, &total);
    g = ex >> 16;
    e = ex & 0xffffu;
    for (int i = i0; i < i1; ++i) {
        const unsigned k = keys[i];
        if (k > T) {
            sel[g + min(e, unsigned(need_eq))] = i;
            ++g;
        } else if (k == T && k) {
            if (e < unsigned(need_eq)) sel[g + e] = i;
            ++e;
        }
    }
    __syncthreads();
    return min(K, int(nvalid));
}

// Score `cpw` candidates per wave.  NS8 = rows per candidate / 8 (rounded up);
// each load slot covers 8 rows (8 lanes x 16 bytes per 128-byte row).
template <int NS8>
__device__ __forceinline__ void score_slice(const PruneParams& p, const int32_t* parents, int64_t L,
                                            const int8_t* __restrict__ k8_bj, const u32x4& qh,
                                            const u32x4& ql, int first, int32_t* __restrict__ out) {
    constexpr int CB = NS8 >= 8 ? 1 : 8 / NS8;     // candidates per batch
    constexpr int NL = CB * NS8;                   // loads per batch
    const int lane = threadIdx.x & 63, row8 = lane >> 3, sl = lane & 7;
    for (int c0 = 0; c0 < p.cpw; c0 += CB) {
        int64_t xs[CB];
#pragma unroll
        for (int c = 0; c < CB; ++c) xs[c] = (c0 + c < p.cpw) ? cand_start(p, parents, first + c0 + c, L) : -1;
        u32x4 v[NL];
        bool ok[NL];
#pragma unroll
        for (int u = 0; u < NL; ++u) {
            const int c = u / NS8, it = u % NS8;
            const int i = it * 8 + row8;
            const int64_t t = xs[c] + int64_t(i) * p.stride;
            ok[u] = xs[c] >= 0 && i < p.nsamp && t < L;
            v[u] = ok[u] ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(k8_bj + t * kHeadDim) + sl)
                         : u32x4{0, 0, 0, 0};
        }
        int best[CB];
#pragma unroll
        for (int c = 0; c < CB; ++c) best[c] = INT32_MIN;
#pragma unroll
        for (int u = 0; u < NL; ++u) {
            int ah = __builtin_amdgcn_sdot4((int)qh.x, (int)v[u].x, 0, false);
            ah = __builtin_amdgcn_sdot4((int)qh.y, (int)v[u].y, ah, false);
            ah = __builtin_amdgcn_sdot4((int)qh.z, (int)v[u].z, ah, false);
            ah = __builtin_amdgcn_sdot4((int)qh.w, (int)v[u].w, ah, false);
            int al = __builtin_amdgcn_sdot4((int)ql.x, (int)v[u].x, 0, false);
            al = __builtin_amdgcn_sdot4((int)ql.y, (int)v[u].y, al, false);
            al = __builtin_amdgcn_sdot4((int)ql.z, (int)v[u].z, al, false);
            al = __builtin_amdgcn_sdot4((int)ql.w, (int)v[u].w, al, false);
            const int s = sum8_i(ah * 64 + al);
            if (ok[u]) best[u / NS8] = max(best[u / NS8], s);
        }
#pragma unroll
        for (int c = 0; c < CB; ++c) {
            const int m = max_groups_i(best[c]);
            if (lane == 0 && c0 + c < p.cpw && first + c0 + c < p.ncand) out[first + c0 + c] = m;
        }
    }
}

// Attended 8-token blocks of one (request, KV head): the kept last-stage
// chunks, the sink [0, sink) and the window [L - window, L), each token once,
// as ascending (block << 8 | token mask) words.
__device__ void build_attended(const PruneParams& p, const int32_t* kept_s, int nk, int64_t L,
                               uint32_t* __restrict__ blocks, int32_t* __restrict__ nblocks,
                               unsigned* tmp) {
    const int tid = threadIdx.x;
    const int64_t s_end = min<int64_t>(p.sink, L);
    const int64_t w0 = p.window > 0 ? max<int64_t>(0, L - p.window) : L;
    const int64_t sb1 = (s_end + 7) >> 3, wb0 = w0 >> 3, wb1 = (L + 7) >> 3;
    const bool merged = wb0 <= sb1;
    const int64_t nr1 = merged ? wb1 : sb1;
    const int64_t nr2 = merged ? 0 : wb1 - wb0;
    const int bpc = p.chunk >> 3;
    const int nmc = nk * bpc;    // candidate middle blocks

    auto kept_block = [&](int64_t blk) -> bool {
        // largest kept start <= 8*blk, then containment
        int lo = 0, hi = nk - 1, pos = -1;
        while (lo <= hi) {
            const int mid = (lo + hi) >> 1;
            if (int64_t(kept_s[mid]) <= blk * 8) { pos = mid; lo = mid + 1; } else { hi = mid - 1; }
        }
        return pos >= 0 && blk * 8 < int64_t(kept_s[pos]) + p.chunk;
    };
    auto mask_of = [&](int64_t blk) -> uint32_t {
        const bool kb = kept_block(blk);
        uint32_t m = 0;
        for (int u = 0; u < 8; ++u) {
            const int64_t t = blk * 8 + u;
            if (t < L && (t < s_end || t >= w0 || kb)) m |= 1u << u;
        }
        return m;
    };

    // middle blocks: kept blocks strictly between the two ranges
    const int per = (nmc + kPruneThreads - 1) / kPruneThreads;
    const int i0 = min(nmc, tid * per), i1 = min(nmc, i0 + per);
    unsigned cnt = 0;
    for (int i = i0; i < i1; ++i) {
        const int64_t blk = (int64_t(kept_s[i / bpc]) >> 3) + (i % bpc);
        cnt += (!merged && blk >= sb1 && blk < wb0 && blk * 8 < L);
    }
    unsigned nmid;
    unsigned pos = block_excl_scan<kPruneThreads>(cnt, tmp, &nmid);
    for (int i = i0; i < i1; ++i) {
        const int64_t blk = (int64_t(kept_s[i / bpc]) >> 3) + (i % bpc);
        if (!merged && blk >= sb1 && blk < wb0 && blk * 8 < L) {
            blocks[nr1 + pos] = uint32_t(blk << 8) | mask_of(blk);
            ++pos;
        }
    }
    for (int64_t r = tid; r < nr1; r += kPruneThreads) blocks[r] = uint32_t(r << 8) | mask_of(r);
    for (int64_t r = tid; r < nr2; r += kPruneThreads) {
        const int64_t blk = wb0 + r;
        blocks[nr1 + nmid + r] = uint32_t(blk << 8) | mask_of(blk);
    }
    if (tid == 0) *nblocks = int32_t(nr1 + nmid + nr2);
}

__global__ __launch_bounds__(kPruneThreads) void sd_prune_stage_kernel(PruneParams p) {
    extern __shared__ uint32_t dyn[];                // keys [ncand] then sel [keep]
    __shared__ int Qlds[kHeadDim];
    __shared__ unsigned hist[256];
    __shared__ unsigned tmp[32];
    __shared__ unsigned last_flag;

    const int j = blockIdx.y, b = blockIdx.z;
    const int bj = b * p.Hkv + j;
    int64_t L = p.lengths[b];
    if (L < 1 || L > p.Lmax) {
        if (p.stage == 0 && blockIdx.x == 0 && threadIdx.x == 0) atomicOr(p.flag, 1);
        L = 0;
    }
    int32_t* kept_bj = p.kept + int64_t(bj) * p.keep_total;

    // group query
    if (p.stage == 0) {
        group_query_codes(p.q + int64_t(b) * p.Hq * kHeadDim, j, p.G, Qlds, nullptr);
        if (blockIdx.x == 0 && threadIdx.x < kHeadDim)
            p.qgroup[int64_t(bj) * kHeadDim + threadIdx.x] = Qlds[threadIdx.x];
    } else {
        if (threadIdx.x < kHeadDim) Qlds[threadIdx.x] = p.qgroup[int64_t(bj) * kHeadDim + threadIdx.x];
        __syncthreads();
    }
    // hi/lo int8 split of this lane's 16 query dims: Q = 64 * hi + lo, lo in [-32, 31]
    const int sl = threadIdx.x & 7;
    u32x4 qh, ql;
    {
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

    const int32_t* parents = p.stage == 0 ? nullptr : kept_bj + p.prev_koff;
    const int8_t* k8_bj = p.k8 + int64_t(bj) * p.Lmax * kHeadDim;
    int32_t* scores_bj = p.scores + int64_t(bj) * p.ncand;
    const int wave = threadIdx.x >> 6;
    const int first = (blockIdx.x * kPruneWaves + wave) * p.cpw;
    const int ns8 = (p.nsamp + 7) >> 3;
    if (ns8 == 1) score_slice<1>(p, parents, L, k8_bj, qh, ql, first, scores_bj);
    else if (ns8 == 2) score_slice<2>(p, parents, L, k8_bj, qh, ql, first, scores_bj);
    else if (ns8 <= 4) score_slice<4>(p, parents, L, k8_bj, qh, ql, first, scores_bj);
    else score_slice<8>(p, parents, L, k8_bj, qh, ql, first, scores_bj);

    if (!arrive_last(p.counter + bj, unsigned(p.nwg), &last_flag)) return;

    // ---- last workgroup of this (request, KV head): select ----
    uint32_t* keys = dyn;
    int* sel = reinterpret_cast<int*>(dyn + p.ncand);
    for (int i = threadIdx.x; i < p.ncand; i += kPruneThreads) {
        const int s = __hip_atomic_load(scores_bj + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        keys[i] = s == INT32_MIN ? 0u : (uint32_t(s) ^ 0x80000000u);
    }
    __syncthreads();
    const int nk = select_top(keys, p.ncand, p.keep, sel, hist, tmp);
    // indices -> starts (reuse sel in place; starts fit int32)
    for (int i = threadIdx.x; i < nk; i += kPruneThreads) sel[i] = int(cand_start(p, parents, sel[i], L));
    __syncthreads();
    for (int i = threadIdx.x; i < p.keep; i += kPruneThreads) kept_bj[p.koff + i] = i < nk ? sel[i] : -1;
    if (p.last_stage) {
        build_attended(p, sel, nk, L, p.blocks + int64_t(bj) * p.max_blocks, p.nblocks + bj, tmp);
    }
}

hipError_t launch_prune_stage(sd_ctx* c, int st, const uint16_t* q, const int8_t* k8, const int32_t* lengths,
                              int32_t* kept, hipStream_t s) {
    PruneParams p{};
    p.q = q;
    p.k8 = k8;
    p.lengths = lengths;
    p.Lmax = c->Lmax;
    p.Hq = c->cfg.num_q_heads;
    p.Hkv = c->cfg.num_kv_heads;
    p.G = c->G;
    p.qgroup = c->qgroup;
    p.kept = kept;
    p.keep_total = c->keep_total;
    p.flag = c->flag;
    p.blocks = c->blocks;
    p.nblocks = c->nblocks;
    p.max_blocks = c->max_blocks;
    p.sink = c->cfg.sink;
    p.window = c->cfg.window;
    const int BH = c->cfg.batch * c->cfg.num_kv_heads;
    const StageGeom& g = c->st[st];
    p.stage = st;
    p.chunk = g.chunk;
    p.stride = g.stride;
    p.keep = g.keep;
    p.nsamp = g.nsamp;
    p.ncand = g.ncand;
    p.koff = g.koff;
    p.cpw = g.per_wg / kPruneWaves;
    p.prev_koff = st ? c->st[st - 1].koff : 0;
    p.ratio = st ? c->st[st - 1].chunk / g.chunk : 1;
    p.scores = c->scores[st];
    p.counter = c->counters + size_t(st) * BH;
    p.nwg = g.nwg;
    p.last_stage = st == c->S - 1;
    const size_t lds = (size_t(g.ncand) + size_t(g.keep)) * 4;
    dim3 grid(g.nwg, c->cfg.num_kv_heads, c->cfg.batch);
    sd_prune_stage_kernel<<<grid, kPruneThreads, lds, s>>>(p);
    return hipGetLastError();
}

}  // namespace sd
