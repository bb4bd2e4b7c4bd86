// LRU cache of 8-token value blocks in device memory, for values that live
// in pinned host memory.
//
// Sources: news article on InfiniteHiP ("韩国通过卸载键值缓存节约英伟达GPU内存，
// 实现18.95倍解码加速"), section "实现 7.24 倍的端到端解码加速" (offloaded KV
// behind an LRU-based cache) and section "解决长上下文推理问题，能通过键值缓存卸载
// 节约 GPU 内存" (the attention kernel reads CPU memory while it runs);
// HCAttention summary page, section 引言 (values held in CPU memory and
// fetched late, for the final aggregation only).
//
// Policy, per (request, KV head): every attended block of a step is touched;
// a block that is not resident takes a free slot (lowest first) or evicts
// the resident block with the smallest (last step used, block id).  The
// recency order is kept explicitly: an array of slots, oldest first, that
// each step rebuilds as [untouched survivors in order] ++ [this step's blocks
// by ascending id], so evicting "the oldest untouched entries" is exactly
// the (last step, block id) rule.  One workgroup per (request, KV head)
// applies a step (after selecting the last stage's kept set and building the
// attended block list, which it publishes for the decode kernel); the decode
// kernel then reads hits from the slot pool and misses straight from host
// memory, writing each missed block into its slot.
//
// The LRU's clock (the step number) lives on the device, one counter per
// (request, KV head) that this kernel reads and advances, so a step
// captured in a graph replays with the right clock.  A slot also records
// how many rows of its block it holds: the rows below the length when it
// was filled.  When the length has grown since, a hit on a block that ends
// at or after the old length is served by reading the block from host
// memory again (a refill); the LRU treats it as the hit it is.
#include "sd_device.h"
#include "sd_internal.h"
#include "sd_select.h"

namespace sd {

constexpr int kLruThreads = 256;

__global__ void sd_vcache_reset_kernel(ValueCache vc, int64_t BH) {
    const int64_t n_page = BH * vc.nblk_max, n_slot = BH * vc.slots;
    const int64_t stride = int64_t(gridDim.x) * blockDim.x;
    const int64_t t0 = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    for (int64_t i = t0; i < n_page; i += stride) vc.page[i] = -1;
    for (int64_t i = t0; i < n_slot; i += stride) {
        vc.slot_block[i] = -1;
        vc.slot_last[i] = -1;
        vc.slot_fill[i] = 0;
    }
    for (int64_t i = t0; i < BH; i += stride) {
        vc.used[i] = 0;
        vc.stepc[i] = 0;
    }
    if (t0 < kVcCounters) vc.counters[t0] = 0;
}

constexpr int kVcBatch = 8;     // LRU entries per batch of loads (per thread)

struct VcStepParams {
    ValueCache vc;
    StageDev last;
    int first_stage;
    int pp_koff;
    const int32_t* last_scores;   // [B][Hkv][last.ncand]
    int32_t* kept;                // [B][Hkv][keep_total]
    int keep_total;
    int32_t* flag;                // bad-length flag (set here when the last stage is given)
    int sink, window;
    const int32_t* lengths;
    int64_t Lmax;
    uint32_t* blocks;             // [B][Hkv][max_blocks]
    int32_t* nblocks;             // [B][Hkv]
    int max_blocks;
    int Hkv;
    // fused last two stages (SELP != 0): P = the stage before the last,
    // scored with every child's last-stage score by its pruning kernel
    StageDev P;
    int p_first;                  // P is the first stage
    int pp_koff_p;                // kept_idx offset of the stage before P
    const int32_t* p_scores;      // [B][Hkv][P.ncand]
    const int32_t* pre;           // [B][Hkv][P.ncand * fuse_rq]
    int fuse_rq;
    int32_t* last_scores_out;     // [B][Hkv][last.ncand]: the last stage's candidate scores (inspection)
};

// Step counters of one (request, KV head) after its LRU step: the clock,
// the used slots, and the hit / miss / refill statistics (sd_get_stats).
__device__ __forceinline__ void vcache_step_stats(const ValueCache& vc, int bj, int32_t step, int used, int nb,
                                                  int nmiss, int nfree, unsigned nref) {
    // refills of this (request, KV head), summed over the block
    if (nref) atomicAdd(reinterpret_cast<unsigned long long*>(vc.counters + 12), (unsigned long long)nref);
    if (nref) atomicAdd(reinterpret_cast<unsigned long long*>(vc.counters + 7 + 4 * (step & 1)), (unsigned long long)nref);
    if (threadIdx.x == 0) {
        vc.stepc[bj] = step + 1;
        vc.used[bj] = used + (nmiss < nfree ? nmiss : nfree);
        const int par = step & 1;
        atomicAdd(reinterpret_cast<unsigned long long*>(vc.counters + 1), (unsigned long long)nb);
        atomicAdd(reinterpret_cast<unsigned long long*>(vc.counters + 2), (unsigned long long)(nb - nmiss));
        atomicAdd(reinterpret_cast<unsigned long long*>(vc.counters + 3), (unsigned long long)nmiss);
        atomicAdd(reinterpret_cast<unsigned long long*>(vc.counters + 4 + 4 * par), (unsigned long long)nb);
        atomicAdd(reinterpret_cast<unsigned long long*>(vc.counters + 5 + 4 * par), (unsigned long long)(nb - nmiss));
        atomicAdd(reinterpret_cast<unsigned long long*>(vc.counters + 6 + 4 * par), (unsigned long long)nmiss);
        if (bj == 0) {
            vc.counters[0] = step + 1;
            const int nxt = (step + 1) & 1;
            vc.counters[4 + 4 * nxt] = 0;
            vc.counters[5 + 4 * nxt] = 0;
            vc.counters[6 + 4 * nxt] = 0;
            vc.counters[7 + 4 * nxt] = 0;
        }
    }
}

// Small caches (FAST: at most kVcOnchipSlots slots and kVcOnchipBlocks
// attended blocks per (request, KV head), unless SD_VCACHE_ONCHIP=0) keep the step's working state on chip: the
// block list and the evicted slots in LDS, each thread's 32 entries of the
// recency order in registers (loaded while the block list is built), the
// slots of this step's blocks in registers, and "touched this step" as an
// LDS bit map of the slots the hits took.  After the select, the only memory
// round trips left are the hits' page-table and fill lookups and, when
// slots are evicted, the blocks those held.  Larger caches take the same
// steps through device memory (slot_last marks the touched slots).
constexpr int kVcFastSlots = kVcOnchipSlots;
constexpr int kVcFastOrd = kVcFastSlots / kLruThreads;     // order entries per thread
constexpr int kVcFastBlocks = kVcOnchipBlocks;
constexpr int kVcFastPer = kVcFastBlocks / kLruThreads;    // attended blocks per thread

// SEL: select code of the last stage, or kGiven when it is reused (read
// from kept_idx).  SELP: select code of the stage before the last when the
// two are fused (that stage's pruning kernel scored the last stage's
// candidates too; both are selected here), else 0.
template <int SEL, bool FAST, int SELP>
__global__ __launch_bounds__(kLruThreads) void sd_vcache_step_kernel(VcStepParams p) {
    extern __shared__ uint32_t dyn[];    // the select(s) (kept_lds_words, or fused_lds_words)
    __shared__ unsigned tmp[32];
    __shared__ uint32_t touchedL[FAST ? kVcFastSlots / 32 : 1];
    __shared__ uint32_t blocksL[FAST ? kVcFastBlocks : 1];
    __shared__ int32_t evictedL[FAST ? kVcFastBlocks : 1];
    __shared__ int32_t ordL[FAST ? kVcFastSlots + kVcFastSlots / 32 : 1];   // entry i at i + i / 32
    const ValueCache& vc = p.vc;
    const int max_blocks = p.max_blocks;
    const int j = blockIdx.x, b = blockIdx.y, bj = b * p.Hkv + j;
    const int32_t step = p.vc.stepc[bj];
    const int64_t BH = int64_t(gridDim.x) * gridDim.y;
    const int tid = threadIdx.x;
    SD_PHASE(4, 0);
    int64_t L = p.lengths[b];
    if (L < 1 || L > p.Lmax) L = 0;

    // last stage's kept set and the attended blocks
    int32_t* kept_bj = p.kept + int64_t(bj) * p.keep_total;
    int* sel = reinterpret_cast<int*>(dyn + p.last.ncand);
    int nk;
    if constexpr (SEL == kGiven) {
        // the last stage is reused: its kept set is read from kept_idx (and
        // no pruning kernel ran this step to flag a bad length)
        if (L == 0 && tid == 0) atomicOr(p.flag, 1);
        nk = given_kept<kLruThreads>(p.last, kept_bj + p.last.koff, L, sel, tmp);
    } else if constexpr (SELP != 0) {
        // fused: select the stage before the last, gather its kept chunks'
        // children's scores, select the last stage; publish both kept sets
        // and the last stage's candidate scores
        const FusedOut fo = kept_two_stages<kLruThreads, SELP, SEL>(
            p.P, p.p_first != 0, p.p_scores + int64_t(bj) * p.P.ncand, p.p_first ? nullptr : kept_bj + p.pp_koff_p,
            p.pre + int64_t(bj) * p.P.ncand * p.fuse_rq, p.fuse_rq, p.last, L, dyn, tmp);
        nk = fo.nq;
        sel = fo.q_starts;
        for (int i = tid; i < p.last.keep; i += kLruThreads) kept_bj[p.last.koff + i] = i < nk ? sel[i] : -1;
        for (int i = tid; i < p.P.keep; i += kLruThreads) kept_bj[p.P.koff + i] = fo.p_starts[i];
        int32_t* sc = p.last_scores_out + int64_t(bj) * p.last.ncand;
        for (int i = tid; i < p.last.ncand; i += kLruThreads) {
            const uint32_t key = fo.q_keys[i];
            sc[i] = key ? int32_t(key) - (1 << 23) : INT32_MIN;
        }
    } else {
        nk = kept_of_stage<kLruThreads, SEL>(p.last, p.first_stage != 0, p.last_scores + int64_t(bj) * p.last.ncand,
                                             p.first_stage ? nullptr : kept_bj + p.pp_koff, L, dyn, tmp);
        for (int i = tid; i < p.last.keep; i += kLruThreads) kept_bj[p.last.koff + i] = i < nk ? sel[i] : -1;
    }
    SD_PHASE(4, 1);
    int32_t* page = vc.page + int64_t(bj) * vc.nblk_max;
    int32_t* sblk = vc.slot_block + int64_t(bj) * vc.slots;
    int32_t* slast = vc.slot_last + int64_t(bj) * vc.slots;
    int32_t* bslot = vc.blk_slot + int64_t(bj) * max_blocks;
    int32_t* evicted = vc.evicted + int64_t(bj) * max_blocks;
    const int32_t* order_old = vc.order + (int64_t(step & 1) * BH + bj) * vc.slots;
    int32_t* order_new = vc.order + (int64_t((step + 1) & 1) * BH + bj) * vc.slots;
    int32_t* sfill = vc.slot_fill + int64_t(bj) * vc.slots;
    const int used = vc.used[bj];
    uint32_t* blocks_bj = p.blocks + int64_t(bj) * max_blocks;
    if constexpr (FAST) {
        // the recency order, loaded while the block list is built
        // (coalesced: entry tid + 256 k, from clamped in-bounds indices, no
        // load under a branch; entries at or past `used` are never read),
        // staged in LDS after the hits' lookups.  The touched map is cleared
        // before build_attended's closing barrier.
        int32_t ov[kVcFastOrd];
#pragma unroll
        for (int k = 0; k < kVcFastOrd; ++k) ov[k] = order_old[min(tid + kLruThreads * k, vc.slots - 1)];
        for (int i = tid; i < kVcFastSlots / 32; i += kLruThreads) touchedL[i] = 0u;
        const int nb = build_attended<kLruThreads>(sel, nk, p.last.chunk, L, p.sink, p.window, blocksL, tmp);
        for (int i = tid; i < nb; i += kLruThreads) blocks_bj[i] = blocksL[i];
        if (tid == 0) p.nblocks[bj] = nb;
        SD_PHASE(4, 2);

        // 1. hits touch their slot (bit map); misses are counted
        const int per = (nb + kLruThreads - 1) / kLruThreads;     // <= kVcFastPer
        const int r0 = min(nb, tid * per), r1 = min(nb, r0 + per);
        uint32_t e[kVcFastPer];
        int32_t bs[kVcFastPer], fv[kVcFastPer];
#pragma unroll
        for (int u = 0; u < kVcFastPer; ++u) e[u] = r0 + u < r1 ? blocksL[r0 + u] : 0u;
#pragma unroll
        for (int u = 0; u < kVcFastPer; ++u) bs[u] = page[e[u] >> 8];
#pragma unroll
        for (int u = 0; u < kVcFastPer; ++u) fv[u] = sfill[max(bs[u], 0)];
        unsigned nm = 0, nref = 0;
#pragma unroll
        for (int u = 0; u < kVcFastPer; ++u) {
            if (r0 + u >= r1) continue;
            const int32_t sv = bs[u];
            if (sv >= 0) {
                atomicOr(&touchedL[sv >> 5], 1u << (sv & 31));
                const int rows = int(min<int64_t>(8, L - 8 * int64_t(e[u] >> 8)));
                if (fv[u] < rows) {
                    sfill[sv] = rows;
                    bs[u] = sv | kVcRefillBit;
                    ++nref;
                }
            } else {
                ++nm;
            }
        }
        // entry i at ordL[i + i / 32]: thread t's entries [32 t, 32 t + 32)
        // then sit 33 words apart, on distinct banks
#pragma unroll
        for (int k = 0; k < kVcFastOrd; ++k) {
            const int i = tid + kLruThreads * k;
            ordL[i + (i >> 5)] = ov[k];
        }
        SD_PHASE(4, 3);
        unsigned nmiss;
        unsigned mrank = block_excl_scan<kLruThreads>(nm, tmp, &nmiss);   // (its barrier completes the map and ordL)
        SD_PHASE(4, 4);
        const int nfree = vc.slots - used;
        const int nevict = int(nmiss) > nfree ? int(nmiss) - nfree : 0;

        // 2. untouched entries keep their order; the oldest `nevict` of them
        //    leave.  Thread t takes entries [32 t, 32 t + 32).
        const int o0 = tid * kVcFastOrd;
        uint32_t umask = 0;
#pragma unroll
        for (int k = 0; k < kVcFastOrd; ++k) {
            ov[k] = ordL[o0 + (tid) + k];             // entry o0 + k at (o0 + k) + (o0 + k) / 32 = 33 t + k
            const int32_t sv = ov[k];
            if (o0 + k < used && !((touchedL[sv >> 5] >> (sv & 31)) & 1u)) umask |= 1u << k;
        }
        unsigned nuntouched;
        unsigned krank = block_excl_scan<kLruThreads>(unsigned(__builtin_popcount(umask)), tmp, &nuntouched);
        SD_PHASE(4, 5);
        // the new order is assembled in ordL (every thread has read its old
        // entries: the scan's barriers) and stored coalesced at the end
        auto pad = [](int i) { return i + (i >> 5); };
        if (nevict > 0) {
            int32_t bv[kVcFastOrd];
#pragma unroll
            for (int k = 0; k < kVcFastOrd; ++k) bv[k] = sblk[((umask >> k) & 1u) ? ov[k] : 0];
#pragma unroll
            for (int k = 0; k < kVcFastOrd; ++k) {
                if (!((umask >> k) & 1u)) continue;
                if (int(krank) < nevict) {
                    page[bv[k]] = -1;
                    evictedL[krank] = ov[k];
                } else {
                    ordL[pad(int(krank) - nevict)] = ov[k];
                }
                ++krank;
            }
        } else {
#pragma unroll
            for (int k = 0; k < kVcFastOrd; ++k)
                if ((umask >> k) & 1u) ordL[pad(int(krank++))] = ov[k];
        }
        __syncthreads();
        SD_PHASE(4, 6);
        const int nsurv = int(nuntouched) - nevict;

        // 3. misses take free slots first (ascending), then the evicted slots
        //    (oldest first); the decode kernel fills them from host memory
#pragma unroll
        for (int u = 0; u < kVcFastPer; ++u) {
            if (r0 + u >= r1 || bs[u] >= 0) continue;
            const int32_t blk = int32_t(e[u] >> 8);
            const int m = int(mrank++);
            const int32_t sl = m < nfree ? used + m : evictedL[m - nfree];
            page[blk] = sl;
            sblk[sl] = blk;
            sfill[sl] = int(min<int64_t>(8, L - 8 * int64_t(blk)));
            bs[u] = sl | kVcMissBit;
        }
        SD_PHASE(4, 7);
        // 4. this step's blocks become the newest entries, ascending by id
#pragma unroll
        for (int u = 0; u < kVcFastPer; ++u) {
            if (r0 + u >= r1) continue;
            bslot[r0 + u] = bs[u];
            ordL[pad(nsurv + r0 + u)] = bs[u] & kVcSlotMask;
        }
        __syncthreads();
        for (int i = tid; i < nsurv + nb; i += kLruThreads) order_new[i] = ordL[pad(i)];
        SD_PHASE(4, 8);
        vcache_step_stats(vc, bj, step, used, nb, int(nmiss), nfree, nref);
        return;
    }
    const int nb = build_attended<kLruThreads>(sel, nk, p.last.chunk, L, p.sink, p.window, blocks_bj, tmp);
    if (tid == 0) p.nblocks[bj] = nb;
    SD_PHASE(4, 2);
    const uint32_t* bl = blocks_bj;

    // 1. hits touch their slot; misses are ranked in block order (ascending id)
    const int per = (nb + kLruThreads - 1) / kLruThreads;
    const int r0 = min(nb, tid * per), r1 = min(nb, r0 + per);
    // (the loops below take kVcBatch entries at a time: their independent
    // loads, then the loads that depend on them, then the updates, so that
    // a batch costs two memory round trips instead of two per entry)
    // (a hit whose slot holds fewer rows than are below the length now is
    // refilled from host memory: only the block holding the old last token
    // can be one, after the length grew)
    unsigned nm = 0, nref = 0;
    for (int b0 = r0; b0 < r1; b0 += kVcBatch) {
        uint32_t e[kVcBatch];
        int32_t sv[kVcBatch], fv[kVcBatch];
#pragma unroll
        for (int u = 0; u < kVcBatch; ++u) e[u] = bl[min(b0 + u, r1 - 1)];    // clamped: no branch
#pragma unroll
        for (int u = 0; u < kVcBatch; ++u) sv[u] = page[e[u] >> 8];
#pragma unroll
        for (int u = 0; u < kVcBatch; ++u) fv[u] = sfill[max(sv[u], 0)];
#pragma unroll
        for (int u = 0; u < kVcBatch; ++u) {
            const int r = b0 + u;
            if (r >= r1) break;
            if (sv[u] >= 0) {
                const int64_t blk = int64_t(e[u] >> 8);
                const int rows = int(min<int64_t>(8, L - 8 * blk));
                slast[sv[u]] = step;
                if (fv[u] < rows) {
                    sfill[sv[u]] = rows;
                    bslot[r] = sv[u] | kVcRefillBit;
                    ++nref;
                } else {
                    bslot[r] = sv[u];
                }
            } else {
                bslot[r] = -1;
                ++nm;
            }
        }
    }
    SD_PHASE(4, 3);
    unsigned nmiss;
    unsigned mrank = block_excl_scan<kLruThreads>(nm, tmp, &nmiss);   // barriers inside
    SD_PHASE(4, 4);
    const int nfree = vc.slots - used;
    const int nevict = int(nmiss) > nfree ? int(nmiss) - nfree : 0;

    // 2. untouched entries keep their order; the oldest `nevict` of them leave
    const int per2 = (used + kLruThreads - 1) / kLruThreads;
    const int i0 = min(used, tid * per2), i1 = min(used, i0 + per2);
    unsigned nu = 0;
    for (int b0 = i0; b0 < i1; b0 += kVcBatch) {
        int32_t sv[kVcBatch], lv[kVcBatch];
#pragma unroll
        for (int u = 0; u < kVcBatch; ++u) sv[u] = order_old[min(b0 + u, i1 - 1)];
#pragma unroll
        for (int u = 0; u < kVcBatch; ++u) lv[u] = slast[sv[u]];
#pragma unroll
        for (int u = 0; u < kVcBatch; ++u) nu += b0 + u < i1 && lv[u] != step;
    }
    unsigned nuntouched;
    unsigned krank = block_excl_scan<kLruThreads>(nu, tmp, &nuntouched);
    SD_PHASE(4, 5);
    for (int b0 = i0; b0 < i1; b0 += kVcBatch) {
        int32_t sv[kVcBatch], lv[kVcBatch], bv[kVcBatch];
#pragma unroll
        for (int u = 0; u < kVcBatch; ++u) sv[u] = order_old[min(b0 + u, i1 - 1)];
#pragma unroll
        for (int u = 0; u < kVcBatch; ++u) {
            lv[u] = slast[sv[u]];
            bv[u] = sblk[sv[u]];
        }
#pragma unroll
        for (int u = 0; u < kVcBatch; ++u) {
            if (b0 + u >= i1 || lv[u] == step) continue;     // past the range, or touched this step
            if (int(krank) < nevict) {
                page[bv[u]] = -1;
                evicted[krank] = sv[u];
            } else {
                order_new[krank - nevict] = sv[u];
            }
            ++krank;
        }
    }
    __syncthreads();
    SD_PHASE(4, 6);
    const int nsurv = int(nuntouched) - nevict;

    // 3. misses take free slots first (ascending), then the evicted slots
    //    (oldest first); the decode kernel fills them from host memory
    for (int r = r0; r < r1; ++r) {
        if (bslot[r] >= 0) continue;
        const int32_t blk = int32_t(bl[r] >> 8);
        const int m = int(mrank++);
        const int32_t s = m < nfree ? used + m : evicted[m - nfree];
        page[blk] = s;
        sblk[s] = blk;
        slast[s] = step;
        sfill[s] = int(min<int64_t>(8, L - 8 * int64_t(blk)));
        bslot[r] = s | kVcMissBit;
    }
    SD_PHASE(4, 7);
    // 4. this step's blocks become the newest entries, ascending by id
    for (int r = r0; r < r1; ++r) order_new[nsurv + r] = bslot[r] & kVcSlotMask;
    SD_PHASE(4, 8);
    vcache_step_stats(vc, bj, step, used, nb, int(nmiss), nfree, nref);
}

SD_PHASE_SETUP(vcache)

hipError_t launch_value_cache_reset(sd_ctx* c, hipStream_t s) {
    const int64_t BH = int64_t(c->cfg.batch) * c->cfg.num_kv_heads;
    sd_vcache_reset_kernel<<<1024, 256, 0, s>>>(c->vc, BH);
    return hipGetLastError();
}

hipError_t launch_value_cache_update(sd_ctx* c, bool given, bool fused, const int32_t* lengths, int32_t* kept,
                                     hipStream_t s, Timing t) {
    VcStepParams p{};
    p.vc = c->vc;
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
    p.lengths = lengths;
    p.Lmax = c->Lmax;
    p.blocks = c->blocks;
    p.nblocks = c->nblocks;
    p.max_blocks = c->max_blocks;
    p.Hkv = c->cfg.num_kv_heads;
    const bool fuse = fused && !given;
    if (fuse) {
        p.P = stage_dev(c, S - 2);
        p.p_first = S == 2;
        p.pp_koff_p = S >= 3 ? c->st[S - 3].koff : 0;
        p.p_scores = c->scores[S - 2];
        p.pre = c->pre;
        p.fuse_rq = c->fuse_rq;
        p.last_scores_out = c->scores[S - 1];
    }
    const size_t lds = size_t(fuse ? fused_lds_words(p.P, p.p_first != 0, p.last, p.fuse_rq)
                                   : kept_lds_words(p.last, p.first_stage != 0)) * 4;
    dim3 grid(c->cfg.num_kv_heads, c->cfg.batch);
    const int sw = select_width(p.last.ncand), sp = fuse ? select_width(p.P.ncand) : 0;
    const dim3 block(kLruThreads);
#define SD_VC(F)                                                                                 \
    if (given) launch(sd_vcache_step_kernel<kGiven, F, 0>, grid, block, lds, s, t, p);           \
    else if (fuse && sp == 4) launch(sd_vcache_step_kernel<4, F, 4>, grid, block, lds, s, t, p);  \
    else if (fuse && sp == 16) launch(sd_vcache_step_kernel<4, F, 16>, grid, block, lds, s, t, p); \
    else if (fuse) launch(sd_vcache_step_kernel<4, F, kSelLds>, grid, block, lds, s, t, p);       \
    else if (sw == 4) launch(sd_vcache_step_kernel<4, F, 0>, grid, block, lds, s, t, p);          \
    else if (sw == 16) launch(sd_vcache_step_kernel<16, F, 0>, grid, block, lds, s, t, p);        \
    else launch(sd_vcache_step_kernel<kSelLds, F, 0>, grid, block, lds, s, t, p);
    if (c->vc_onchip) {
        SD_VC(true)
    } else {
        SD_VC(false)
    }
#undef SD_VC
    return hipGetLastError();
}

}  // namespace sd
