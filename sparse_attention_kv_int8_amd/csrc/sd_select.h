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

// LDS words the select needs besides keys [n] and sel [K + 1].
__host__ __device__ inline int select_cand_words(int n, int K) {
    const int groups = (n + 1022) / 1023;
    return groups > 1 ? groups * (K + 1) + groups : 0;
}

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

// ------------------------------------------------------------------------
// Exact top-K select.
//
// Keys are score + 2^23 (a chunk score satisfies |S| <= 4 * 127 * 127 * 128
// < 2^23, so a key lies in [1, 2^24)), with 0 meaning "no candidate"; a
// larger key is better and equal keys go to the lower index.  The
// threshold T (the K-th largest key) is built two bits per round from the
// top: three candidate thresholds are counted per lane in VALU, the counts
// packed into 16-bit fields and summed across the wave with DPP, and the
// largest threshold whose count reaches K is kept.  Keys > T are kept, and
// of the keys equal to T the lowest indices, K - #(keys > T) of them.  One
// wave does the whole search: no barrier and no LDS atomics (both are slow
// on this chip compared with DPP).
// ------------------------------------------------------------------------
constexpr int kSelGroup = 1023;              // keys one wave selects from (<= 16 per lane)
constexpr int kKeyBits = 24;

__device__ __forceinline__ uint32_t score_key(int s) {
    return s == INT32_MIN ? 0u : uint32_t(s + (1 << 23));
}

// Wave-wide sum of a value whose 16-bit fields stay below 2^16.
__device__ __forceinline__ unsigned wave_sum_packed(unsigned v) { return wave_sum_u(v); }

// One wave: top-K of m keys key(i) = keys[idx ? idx[i] : i], m <= min(64 E, 1023).
// Lane l owns the contiguous positions [l*E, l*E + E).  Writes the kept
// positions i (ascending) to out[0..kept) (out has K + 1 slots; slot K is
// scratch); returns kept = min(K, #valid).
template <int E>
__device__ __forceinline__ int wave_select_e(const uint32_t* keys, const int* idx, int m, int K, int* out) {
    const int lane = threadIdx.x & 63;
    uint32_t kk[E];
    unsigned nv = 0;
#pragma unroll
    for (int u = 0; u < E; ++u) {
        const int i = lane * E + u;
        kk[u] = i < m ? keys[idx ? idx[i] : i] : 0u;
        nv += kk[u] != 0u;
    }
    const int nvalid = int(wave_sum_u(nv));
    uint32_t T = 0;
    int need_eq = 0;
    if (nvalid > K) {
        // Round: thresholds prefix + {1,2,3} << b.  For a key, d = number of
        // them it reaches = clamp((key - prefix) >> b, 0, 3); its packed
        // contribution 0x100401 >> (30 - 10 d) adds 1 to each of the d lowest
        // 10-bit fields (fields: reaches c1, c2, c3).  Wave sums of a field
        // stay below 2^10 because m <= 1023.
        uint32_t prefix = 0;
        for (int b = kKeyBits - 2; b >= 0; b -= 2) {
            unsigned acc = 0;
#pragma unroll
            for (int u = 0; u < E; ++u) {
                const int d = min(max((int(kk[u]) - int(prefix)) >> b, 0), 3);
                acc += 0x100401u >> (30 - 10 * d);
            }
            acc = wave_sum_u(acc);
            const int n1 = int(acc & 0x3ffu), n2 = int((acc >> 10) & 0x3ffu), n3 = int(acc >> 20);
            prefix += n3 >= K ? (3u << b) : n2 >= K ? (2u << b) : n1 >= K ? (1u << b) : 0u;
        }
        T = prefix;
        unsigned gl = 0;
#pragma unroll
        for (int u = 0; u < E; ++u) gl += kk[u] > T ? 1u : 0u;
        need_eq = K - int(wave_sum_u(gl));
    }
    // ordered compaction: (count of keys > T, count of keys == T) per lane, scanned
    unsigned g = 0, e = 0;
#pragma unroll
    for (int u = 0; u < E; ++u) { g += kk[u] > T; e += (kk[u] == T) && kk[u]; }
    const unsigned packed = (g << 16) | e;
    const unsigned ex = wave_incl_scan(packed) - packed;
    g = ex >> 16;
    e = ex & 0xffffu;
    const unsigned neq = unsigned(need_eq);
#pragma unroll
    for (int u = 0; u < E; ++u) {
        const bool gt = kk[u] > T;
        const bool eq = (kk[u] == T) && kk[u];
        const unsigned pos = gt ? g + min(e, neq) : (eq && e < neq) ? g + e : unsigned(K);
        out[pos] = lane * E + u;          // non-kept keys land in the scratch slot K
        g += gt;
        e += eq;
    }
    return min(K, nvalid);
}

__device__ __forceinline__ int wave_select(const uint32_t* keys, const int* idx, int m, int K, int* out) {
    if (m <= 64) return wave_select_e<1>(keys, idx, m, K, out);
    if (m <= 128) return wave_select_e<2>(keys, idx, m, K, out);
    if (m <= 256) return wave_select_e<4>(keys, idx, m, K, out);
    if (m <= 512) return wave_select_e<8>(keys, idx, m, K, out);
    return wave_select_e<16>(keys, idx, m, K, out);      // m <= 1023
}

// Block-level: top-K of n keys in LDS (n <= 16 * kSelGroup).  Groups of
// kSelGroup keys are reduced to their own top-K by the waves in parallel
// (exact: a key among the global top K is among its group's top K under the
// same order); one wave then selects from the groups' survivors.  sel
// (K + 1 ints) receives the kept indices ascending.  cand: LDS,
// select_cand_words(n, K) ints.
template <int NT>
__device__ int select_top(const uint32_t* keys, int n, int K, int* sel, int* cand, unsigned* tmp) {
    constexpr int NW = NT / kWave;
    const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int ngroups = (n + kSelGroup - 1) / kSelGroup;
    int kept;
    if (K >= n) {
        // every valid key is kept: ordered compaction
        const int per = (n + NT - 1) / NT;
        const int i0 = min(n, int(threadIdx.x) * per), i1 = min(n, i0 + per);
        unsigned c = 0;
        for (int i = i0; i < i1; ++i) c += keys[i] != 0u;
        unsigned total;
        unsigned pos = block_excl_scan<NT>(c, tmp, &total);
        for (int i = i0; i < i1; ++i)
            if (keys[i]) sel[pos++] = i;
        __syncthreads();
        kept = int(total);
    } else if (ngroups <= 1) {
        if (wid == 0) {
            const int r = wave_select(keys, nullptr, n, K, sel);
            if (lane == 0) tmp[0] = unsigned(r);
        }
        __syncthreads();
        kept = int(tmp[0]);
    } else {
        int* counts = cand + ngroups * (K + 1);     // [ngroups]
        for (int g = wid; g < ngroups; g += NW) {
            const int base = g * kSelGroup;
            const int m = min(kSelGroup, n - base);
            int* out = cand + g * (K + 1);
            const int r = wave_select(keys + base, nullptr, m, K, out);
            for (int i = lane; i < r; i += kWave) out[i] += base;
            if (lane == 0) counts[g] = r;
        }
        __syncthreads();
        if (wid == 0) {
            // compact the survivors in group order (ascending index) in place
            int off = 0;
            for (int g = 0; g < ngroups; ++g) {
                const int r = counts[g];
                for (int i = lane; i < r; i += kWave) cand[off + i] = cand[g * (K + 1) + i];
                off += r;
                __builtin_amdgcn_wave_barrier();
            }
            const int r = wave_select(keys, cand, off, K, sel);
            // positions -> indices
            for (int i = lane; i < r; i += kWave) sel[i] = cand[sel[i]];
            if (lane == 0) tmp[0] = unsigned(r);
        }
        __syncthreads();
        kept = int(tmp[0]);
    }
    return kept;
}

// Kept set of stage `st` for one (request, KV head), from that stage's
// scores (global, INT32_MIN = no candidate): sel[0..nk) receives the kept
// chunk starts, ascending.  `parents` are the kept starts of the stage
// before (global or LDS; unused for the first stage).  keys: LDS [ncand];
// sel: LDS [keep + 1]; cand: LDS [select_cand_words(ncand, keep)].
template <int NT>
__device__ int kept_of_stage(const StageDev& st, bool first_stage, const int32_t* scores_bj,
                             const int32_t* parents, int64_t L, uint32_t* keys, int* sel, int* cand,
                             unsigned* tmp) {
    for (int i = threadIdx.x; i < st.ncand; i += NT) {
        keys[i] = score_key(scores_bj[i]);
    }
    __syncthreads();
    const int nk = select_top<NT>(keys, st.ncand, st.keep, sel, cand, tmp);
    for (int i = threadIdx.x; i < nk; i += NT) sel[i] = int(cand_start(st, first_stage, parents, sel[i], L));
    __syncthreads();
    return nk;
}

// Attended 8-token blocks of one (request, KV head): the kept last-stage
// chunks (starts kept_s[0..nk), ascending, chunk a multiple of 8), the sink
// [0, sink) and the window [L - window, L), each token once, as ascending
// (block << 8 | token mask) words.  Returns the count (the same in every
// thread); the list is complete after the closing barrier.
//
// Layout of the output: sink-range blocks, then the kept blocks strictly
// between the two ranges, then the window-range blocks (one merged range
// when sink and window touch).  The kept blocks form a sorted list (index
// q -> block kept_s[q / bpc] / 8 + q % bpc), so the middle ones are the
// contiguous slice between two binary searches.
template <int NT>
__device__ int build_attended(const int32_t* kept_s, int nk, int chunk, int64_t L, int sink, int window,
                              uint32_t* blocks, unsigned* tmp) {
    (void)tmp;
    const int tid = threadIdx.x;
    const int64_t s_end = min<int64_t>(sink, L);
    const int64_t w0 = window > 0 ? max<int64_t>(0, L - window) : L;
    const int64_t sb1 = (s_end + 7) >> 3, wb1 = (L + 7) >> 3;
    const int64_t wb0 = window > 0 ? (w0 >> 3) : wb1;
    const bool merged = wb0 <= sb1;
    const int64_t nr1 = merged ? wb1 : sb1;
    const int64_t nr2 = merged ? 0 : wb1 - wb0;
    const int bpc = chunk >> 3;
    const int nq = nk * bpc;
    auto blk_at = [&](int q) -> int64_t { return (int64_t(kept_s[q / bpc]) >> 3) + (q % bpc); };
    auto lower = [&](int64_t v) -> int {     // first q with blk_at(q) >= v
        int lo = 0, hi = nq;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (blk_at(mid) < v) lo = mid + 1; else hi = mid;
        }
        return lo;
    };
    auto kept_block = [&](int64_t blk) -> bool {
        const int q = lower(blk);
        return q < nq && blk_at(q) == blk;
    };
    auto valid_mask = [&](int64_t blk) -> uint32_t {
        const int64_t over = blk * 8 + 8 - L;
        return over <= 0 ? 0xffu : (over >= 8 ? 0u : (0xffu >> over));
    };
    auto range_mask = [&](int64_t blk) -> uint32_t {
        uint32_t m = 0;
        for (int u = 0; u < 8; ++u) {
            const int64_t t = blk * 8 + u;
            if (t < s_end || t >= w0) m |= 1u << u;
        }
        m &= valid_mask(blk);
        if (m != valid_mask(blk) && kept_block(blk)) m = valid_mask(blk);
        return m;
    };
    int q0 = 0, q1 = 0;
    if (!merged) {
        q0 = lower(sb1);
        q1 = lower(wb0);
    }
    const int64_t nmid = q1 - q0;
    for (int q = q0 + tid; q < q1; q += NT) {
        const int64_t blk = blk_at(q);
        blocks[nr1 + (q - q0)] = uint32_t(blk << 8) | valid_mask(blk);
    }
    for (int64_t r = tid; r < nr1; r += NT) blocks[r] = uint32_t(r << 8) | range_mask(r);
    for (int64_t r = tid; r < nr2; r += NT) blocks[nr1 + nmid + r] = uint32_t((wb0 + r) << 8) | range_mask(wb0 + r);
    __syncthreads();
    return int(nr1 + nmid + nr2);
}

}  // namespace sd
