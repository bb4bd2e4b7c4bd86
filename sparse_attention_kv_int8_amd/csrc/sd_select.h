// Exact per-(request, KV head) top-K select and the attended block list.
//
// Every workgroup that needs a stage's kept set recomputes it from that
// stage's candidate scores (a few KiB, cache resident): the selection is
// deterministic, so all workgroups of a (request, KV head) agree, and no
// cross-workgroup counter or fence is needed (device-scope atomics on one
// address serialise at roughly 0.1 us each on this chip, which made a
// "last workgroup" hand-off far slower than recomputing).
//
// Selection order: score descending, then candidate index (= chunk start)
// ascending, following the top-K chunk rule of the news article on
// InfiniteHiP, section "实现 7.24 倍的端到端解码加速", with ties to the lower
// start.  The attended set adds the sink and recent window of page
// "KV Cache 与长上下文推理", section "KV Cache 压缩技术" (StreamingLLM).
#pragma once

#include "sd_device.h"
#include "sd_internal.h"

namespace sd {

// Start of candidate i of a stage (token position), or -1 if it does not
// exist.  Stage 0 candidates are i * chunk; later ones are children of the
// previous stage's kept starts `parents` (ascending, -1 padded).
__device__ __forceinline__ int64_t cand_start(const StageDev& st, bool first_stage, const int32_t* parents,
                                              int i, int64_t L) {
    if (i >= st.ncand) return -1;
    int64_t x;
    if (first_stage) {
        x = int64_t(i) * st.chunk;
    } else {
        const int par = parents[i / st.ratio];
        if (par < 0) return -1;
        x = int64_t(par) + int64_t(i % st.ratio) * st.chunk;
    }
    return x < L ? x : -1;
}

// Exact top-K of n keys (0 = no candidate; otherwise larger is better, ties
// to the lower index).  keys: LDS [n].  Writes the kept indices ascending to
// sel[0..kept) and returns kept = min(K, #valid).  All NT threads call it.
// hist: NT/64 * 256 words of LDS (one histogram per wave); tmp: 32 words.
//
// Radix select over the bits in which the valid keys differ, 8 bits per
// pass from the top: each pass histograms the keys that share the prefix
// found so far and picks the digit at which the count of larger keys
// reaches K.  The threshold key T and the number of keys equal to T to keep
// (lowest indices first) then drive one ordered compaction.
template <int NT>
__device__ int select_top(const uint32_t* keys, int n, int K, int* sel, unsigned* hist, unsigned* tmp) {
    constexpr int NW = NT / kWave;
    static_assert(3 * NW <= 28, "tmp layout: 3 words per wave below the digit slots 28/29");
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    unsigned cnt = 0, kmn = 0xffffffffu, kmx = 0;
    for (int i = tid; i < n; i += NT) {
        const unsigned k = keys[i];
        if (k) { ++cnt; kmn = min(kmn, k); kmx = max(kmx, k); }
    }
    cnt = wave_sum_u(cnt);
    kmn = wave_min_u(kmn);
    kmx = wave_max_u(kmx);
    if (lane == 0) { tmp[wid] = cnt; tmp[NW + wid] = kmn; tmp[2 * NW + wid] = kmx; }
    __syncthreads();
    unsigned nvalid = 0;
    kmn = 0xffffffffu;
    kmx = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) { nvalid += tmp[w]; kmn = min(kmn, tmp[NW + w]); kmx = max(kmx, tmp[2 * NW + w]); }
    __syncthreads();

    unsigned T = 0;          // threshold key
    int need_eq = 0;         // keys equal to T that are kept (lowest indices first)
    if (int(nvalid) > K) {
        const unsigned diff = kmx ^ kmn;
        int bits = diff ? 32 - __clz(diff) : 0;      // low bits in which keys differ
        unsigned prefix = bits >= 32 ? 0u : (kmx >> bits) << bits;
        int remaining = K;
        unsigned* my_hist = hist + wid * 256;
        while (bits > 0) {
            const int w = bits < 8 ? bits : 8;
            const int shift = bits - w;
            for (int i = tid; i < NW * 256; i += NT) hist[i] = 0;
            __syncthreads();
            const unsigned hi_mask = bits >= 32 ? 0u : ~((1u << bits) - 1u);
            const unsigned want = prefix & hi_mask, dmask = (1u << w) - 1u;
            for (int i = tid; i < n; i += NT) {
                const unsigned k = keys[i];
                if (k && (k & hi_mask) == want) atomicAdd(my_hist + ((k >> shift) & dmask), 1u);
            }
            __syncthreads();
            if (wid == 0) {
                // lane l owns bins 255-4l .. 252-4l (descending digit order)
                unsigned h[4], s4 = 0;
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    unsigned c = 0;
#pragma unroll
                    for (int v = 0; v < NW; ++v) c += hist[v * 256 + 255 - 4 * lane - u];
                    h[u] = c;
                    s4 += c;
                }
                const unsigned incl = wave_incl_scan(s4), excl = incl - s4;
                if (excl < unsigned(remaining) && unsigned(remaining) <= incl) {
                    unsigned c = excl;
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        if (c + h[u] >= unsigned(remaining)) {
                            tmp[28] = unsigned(255 - 4 * lane - u);
                            tmp[29] = c;
                            break;
                        }
                        c += h[u];
                    }
                }
            }
            __syncthreads();
            const unsigned dd = tmp[28], above = tmp[29];
            remaining -= int(above);
            prefix |= dd << shift;
            bits = shift;
        }
        T = prefix;
        need_eq = remaining;
    }
    // Compaction in index order: thread t owns the contiguous range [i0, i1).
    const int per = (n + NT - 1) / NT;
    const int i0 = min(n, tid * per), i1 = min(n, i0 + per);
    unsigned g = 0, e = 0;
    for (int i = i0; i < i1; ++i) {
        const unsigned k = keys[i];
        g += k > T;
        e += (k == T) && k;
    }
    unsigned total;
    const unsigned ex = block_excl_scan<NT>((g << 16) | e, tmp, &total);
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

// Kept set of stage `st` for one (request, KV head), from that stage's
// scores (global, INT32_MIN = no candidate): sel[0..nk) receives the kept
// chunk starts, ascending.  `parents` are the kept starts of the stage
// before (global or LDS; unused for the first stage).  keys: LDS [ncand].
template <int NT>
__device__ int kept_of_stage(const StageDev& st, bool first_stage, const int32_t* scores_bj,
                             const int32_t* parents, int64_t L, uint32_t* keys, int* sel, unsigned* hist,
                             unsigned* tmp) {
    for (int i = threadIdx.x; i < st.ncand; i += NT) {
        const int s = scores_bj[i];
        keys[i] = s == INT32_MIN ? 0u : (uint32_t(s) ^ 0x80000000u);
    }
    __syncthreads();
    const int nk = select_top<NT>(keys, st.ncand, st.keep, sel, hist, tmp);
    for (int i = threadIdx.x; i < nk; i += NT) sel[i] = int(cand_start(st, first_stage, parents, sel[i], L));
    __syncthreads();
    return nk;
}

// Attended 8-token blocks of one (request, KV head): the kept last-stage
// chunks (starts kept_s[0..nk), ascending, chunk a multiple of 8), the sink
// [0, sink) and the window [L - window, L), each token once, as ascending
// (block << 8 | token mask) words.  Returns the count; all NT threads call.
template <int NT>
__device__ int build_attended(const int32_t* kept_s, int nk, int chunk, int64_t L, int sink, int window,
                              uint32_t* blocks, unsigned* tmp) {
    const int tid = threadIdx.x;
    const int64_t s_end = min<int64_t>(sink, L);
    const int64_t w0 = window > 0 ? max<int64_t>(0, L - window) : L;
    const int64_t sb1 = (s_end + 7) >> 3, wb1 = (L + 7) >> 3;
    const int64_t wb0 = window > 0 ? (w0 >> 3) : wb1;
    const bool merged = wb0 <= sb1;
    const int64_t nr1 = merged ? wb1 : sb1;
    const int64_t nr2 = merged ? 0 : wb1 - wb0;
    const int bpc = chunk >> 3;
    const int nmc = nk * bpc;

    auto kept_block = [&](int64_t blk) -> bool {
        int lo = 0, hi = nk - 1, pos = -1;
        while (lo <= hi) {
            const int mid = (lo + hi) >> 1;
            if (int64_t(kept_s[mid]) <= blk * 8) { pos = mid; lo = mid + 1; } else { hi = mid - 1; }
        }
        return pos >= 0 && blk * 8 < int64_t(kept_s[pos]) + chunk;
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
    auto is_mid = [&](int64_t blk) { return !merged && blk >= sb1 && blk < wb0 && blk * 8 < L; };

    const int per = (nmc + NT - 1) / NT;
    const int i0 = min(nmc, tid * per), i1 = min(nmc, i0 + per);
    unsigned cnt = 0;
    for (int i = i0; i < i1; ++i) cnt += is_mid((int64_t(kept_s[i / bpc]) >> 3) + (i % bpc));
    unsigned nmid;
    unsigned pos = block_excl_scan<NT>(cnt, tmp, &nmid);
    for (int i = i0; i < i1; ++i) {
        const int64_t blk = (int64_t(kept_s[i / bpc]) >> 3) + (i % bpc);
        if (is_mid(blk)) blocks[nr1 + pos++] = uint32_t(blk << 8) | mask_of(blk);
    }
    for (int64_t r = tid; r < nr1; r += NT) blocks[r] = uint32_t(r << 8) | mask_of(r);
    for (int64_t r = tid; r < nr2; r += NT) blocks[nr1 + nmid + r] = uint32_t((wb0 + r) << 8) | mask_of(wb0 + r);
    __syncthreads();
    return int(nr1 + nmid + nr2);
}

}  // namespace sd
