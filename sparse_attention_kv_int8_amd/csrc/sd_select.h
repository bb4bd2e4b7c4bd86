// Exact per-(request, KV head) top-K select and the attended block list.
//
// A stage's kept set is selected by every workgroup of the next kernel that
// needs it (the next pruning kernel, or the decode kernel's kept-chunk
// splits for the last stage), redundantly, from the stage's scores (a few
// KiB): the selection is deterministic, so all workgroups of a (request, KV
// head) agree, and no workgroup waits for another.
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

// ------------------------------------------------------------------------
// Exact top-K select.
//
// Keys are score + 2^23 (a chunk score satisfies |S| <= 4 * 127 * 127 * 128
// < 2^23, so a key lies in [1, 2^24)), with 0 meaning "no candidate"; a
// larger key is better and equal keys go to the lower index.
//
// Radix select on 8-bit digits.  Keys are rebased to k - min + 1 (the
// valid count, min and max come with the load of the keys into LDS); each
// round counts the digit (k - lo) >> sh of the keys still undecided (those
// in the bucket [lo, lo + 2^wl)) into an LDS histogram of 256 bins, and
// wave 0 scans the bins from the top digit down (four per lane, one wave
// scan) for the digit that holds the K-th key: keys above it are kept, keys
// below it dropped, and the bucket narrows to that digit.  At most three
// rounds resolve 24 bits, two barriers each; a round whose digit holds
// exactly the keys still wanted ends the search.  The compaction keeps, in
// index order, every key above the threshold T and the first need_eq keys
// equal to it.
// ------------------------------------------------------------------------
__device__ __forceinline__ uint32_t score_key(int s) {
    return s == INT32_MIN ? 0u : uint32_t(s + (1 << 23));
}

// Compares of 4 keys against a wave-uniform threshold, each into its own
// scalar register pair (the lanes that pass), issued back to back: a
// compare's mask is ready for its scalar popcount only some 30 cycles
// later, so the compares of a block overlap that latency.
#define SD_CMP(op, d, v, t) "v_cmp_" op "_u32_e64 %" #d ", %" #v ", %" #t "\n\t"
__device__ __forceinline__ void cmp4_ge(const uint32_t* k, uint32_t t, uint64_t* m) {
    asm(SD_CMP("ge", 0, 4, 8) SD_CMP("ge", 1, 5, 8) SD_CMP("ge", 2, 6, 8) SD_CMP("ge", 3, 7, 8)
        : "=&s"(m[0]), "=&s"(m[1]), "=&s"(m[2]), "=&s"(m[3])
        : "v"(k[0]), "v"(k[1]), "v"(k[2]), "v"(k[3]), "s"(__builtin_amdgcn_readfirstlane(t)));
}
__device__ __forceinline__ void cmp4_gt(const uint32_t* k, uint32_t t, uint64_t* m) {
    asm(SD_CMP("gt", 0, 4, 8) SD_CMP("gt", 1, 5, 8) SD_CMP("gt", 2, 6, 8) SD_CMP("gt", 3, 7, 8)
        : "=&s"(m[0]), "=&s"(m[1]), "=&s"(m[2]), "=&s"(m[3])
        : "v"(k[0]), "v"(k[1]), "v"(k[2]), "v"(k[3]), "s"(__builtin_amdgcn_readfirstlane(t)));
}
#undef SD_CMP
__device__ __forceinline__ int popc(uint64_t m) { return __builtin_popcountll(m); }
// Set bits of m in lanes below this one.
__device__ __forceinline__ unsigned below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi(unsigned(m >> 32), __builtin_amdgcn_mbcnt_lo(unsigned(m), 0u));
}

// LDS scratch of a select: 256 histogram bins, then the boundary found by a
// round (digit, keys above it, keys in it).
constexpr int kRadixWords = 256 + 4;

// Valid count, minimum and maximum of a stage's select keys.
struct KeyStats {
    int nvalid;
    uint32_t kmin, kmax;
};

// Per-thread (count, min, max) -> workgroup totals, through xch[0..4 NW);
// contains the barrier that also orders the caller's LDS stores before the
// select.
template <int NT>
__device__ __forceinline__ KeyStats block_key_stats(unsigned nv, uint32_t kmin, uint32_t kmax, unsigned* xch) {
    constexpr int NW = NT / kWave;
    const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
    nv = wave_sum_u(nv);
    kmin = wave_min_u(kmin);
    kmax = wave_max_u(kmax);
    if (lane == 0) {
        xch[wid * 4] = nv;
        xch[wid * 4 + 1] = kmin;
        xch[wid * 4 + 2] = kmax;
    }
    __syncthreads();
    KeyStats st{0, 0xffffffffu, 0u};
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        st.nvalid += int(xch[w * 4]);
        st.kmin = min(st.kmin, xch[w * 4 + 1]);
        st.kmax = max(st.kmax, xch[w * 4 + 2]);
    }
    return st;
}

// Loads n chunk scores into LDS as select keys, clears the histogram of the
// select scratch `cand` (kRadixWords words), and returns the KeyStats; also
// stages npar ints `parents` (the previous stage's kept starts) into `par`
// (LDS).  Both are read from the L2.  The parents' loads and the
// first kLoadBatch scores of every thread are issued before any of them is
// waited for, so up to 2048 candidates cost one memory round trip (the loads of a
// wave complete in issue order: a load-wait-store loop would pay one round
// trip per iteration).  xch: 16 words.  Ends with a barrier.
constexpr int kLoadBatch = 8;
constexpr int kParBatch = 2;

template <int NT>
__device__ KeyStats load_keys(const int32_t* scores, int n, uint32_t* keys, uint32_t* cand, unsigned* xch,
                              const int32_t* parents = nullptr, int npar = 0, int* par = nullptr) {
    static_assert(NT >= 256, "one thread per histogram bin");
    const int tid = threadIdx.x;
    if (tid < 256) cand[tid] = 0u;
    unsigned nv = 0, kmin = 0xffffffffu, kmax = 0;
    auto put = [&](int i, int32_t sc) {
        const uint32_t k = score_key(sc);
        keys[i] = k;
        nv += k != 0u;
        kmin = min(kmin, k ? k : 0xffffffffu);
        kmax = max(kmax, k);
    };
    int32_t pv[kParBatch];
#pragma unroll
    for (int u = 0; u < kParBatch; ++u) {
        const int i = tid + u * NT;
        pv[u] = i < npar ? parents[i] : -1;
    }
    for (int i0 = tid; i0 < n; i0 += kLoadBatch * NT) {
        int32_t sv[kLoadBatch];
#pragma unroll
        for (int u = 0; u < kLoadBatch; ++u) {
            const int i = i0 + u * NT;
            sv[u] = i < n ? scores[i] : INT32_MIN;
        }
        if (i0 == tid) {
#pragma unroll
            for (int u = 0; u < kParBatch; ++u)
                if (tid + u * NT < npar) par[tid + u * NT] = pv[u];
        }
#pragma unroll
        for (int u = 0; u < kLoadBatch; ++u)
            if (i0 + u * NT < n) put(i0 + u * NT, sv[u]);
    }
    if (n <= tid) {                              // no score of this thread: its parents still go in
#pragma unroll
        for (int u = 0; u < kParBatch; ++u)
            if (tid + u * NT < npar) par[tid + u * NT] = pv[u];
    }
    for (int i = tid + kParBatch * NT; i < npar; i += NT) par[i] = parents[i];
    return block_key_stats<NT>(nv, kmin, kmax, xch);
}

// Top-K of n keys in LDS (K < n), with their KeyStats and a cleared
// histogram.  S > 0: each lane holds S keys in registers (n <= NW * 64 * S);
// S == 0: the keys stay in LDS and every pass reads them, 4 slots at a time.
// Wave w covers positions [w P, (w + 1) P) slot-major (slot u of lane l is
// position w P + 64 u + l), so ascending position is wave-major.  Writes the
// kept positions, ascending, to sel; xch[4 NW, 6 NW) carries the per-wave
// counts of the compaction.  Ends with a barrier; returns min(K, #valid).
template <int NT, int S>
__device__ int radix_select(const uint32_t* keys, int n, int K, int* sel, uint32_t* hist, unsigned* xch,
                            const KeyStats ks) {
    static_assert(NT == 256 && S % 4 == 0, "four waves, one histogram bin per thread, blocks of 4 slots");
    constexpr int NW = NT / kWave;
    const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
    unsigned* bnd = hist + 256;
    const uint32_t gmin = ks.kmin;
    auto rk = [&](uint32_t k) -> uint32_t { return k ? k - gmin + 1u : 0u; };
    const int nblk = S > 0 ? S / 4 : (((n + NW - 1) / NW + 63) / 64 + 3) / 4;
    const int base = wid * nblk * 256;
    uint32_t kk[S > 0 ? S : 4];
    if constexpr (S > 0) {
#pragma unroll
        for (int u = 0; u < S; ++u) {
            const int i = base + 64 * u + lane;
            kk[u] = rk(i < n ? keys[i] : 0u);
        }
    }
    // f(u0, k4) for every block of 4 slots, with the rebased keys
    auto blocks = [&](auto&& f) {
        if constexpr (S > 0) {
#pragma unroll
            for (int u0 = 0; u0 < S; u0 += 4) f(u0, kk + u0);
        } else {
#pragma unroll 1
            for (int u0 = 0; u0 < nblk * 4; u0 += 4) {
                uint32_t k4[4];
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int i = base + 64 * (u0 + v) + lane;
                    k4[v] = rk(i < n ? keys[i] : 0u);
                }
                f(u0, k4);
            }
        }
    };
    uint32_t T = 0;
    int need_eq = 0;
    if (ks.nvalid > K) {
        const uint32_t range = ks.kmax - gmin + 1u;     // rebased keys lie in [1, range]
        int wl = 32 - __builtin_clz(range);             // bucket [lo, lo + 2^wl)
        int sh = wl > 8 ? wl - 8 : 0;
        uint32_t lo = 0;
        int want = K;
        for (;;) {
            const uint32_t lo1 = lo ? lo : 1u, span = 1u << wl;
            blocks([&](int, const uint32_t* k4) {
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    if (k4[v] >= lo1 && k4[v] - lo < span) atomicAdd(&hist[(k4[v] - lo) >> sh], 1u);
            });
            __syncthreads();
            if (wid == 0) {
                // lane l: digits 255 - 4 l down to 252 - 4 l, cleared for the next round
                const int b0 = 252 - 4 * lane;
                const unsigned c3 = hist[b0 + 3], c2 = hist[b0 + 2], c1 = hist[b0 + 1], c0 = hist[b0];
                hist[b0 + 3] = 0u;
                hist[b0 + 2] = 0u;
                hist[b0 + 1] = 0u;
                hist[b0] = 0u;
                const unsigned s4 = c0 + c1 + c2 + c3;
                const unsigned incl = wave_incl_scan(s4);
                unsigned e = incl - s4;                 // keys in higher digits
                const unsigned w = unsigned(want);
                if (e < w && incl >= w) {               // exactly one lane
                    unsigned d, cd;
                    if (e + c3 >= w) {
                        d = b0 + 3;
                        cd = c3;
                    } else if (e + c3 + c2 >= w) {
                        e += c3;
                        d = b0 + 2;
                        cd = c2;
                    } else if (e + c3 + c2 + c1 >= w) {
                        e += c3 + c2;
                        d = b0 + 1;
                        cd = c1;
                    } else {
                        e += c3 + c2 + c1;
                        d = b0;
                        cd = c0;
                    }
                    bnd[0] = d;
                    bnd[1] = e;
                    bnd[2] = cd;
                }
            }
            __syncthreads();
            const uint32_t d = bnd[0];
            const int above = int(bnd[1]), cd = int(bnd[2]);
            want -= above;
            lo += d << sh;
            if (cd == want) {            // the whole digit is kept
                T = lo ? lo - 1u : 0u;
                break;
            }
            if (sh == 0) {               // a single value: ties
                T = lo;
                need_eq = want;
                break;
            }
            wl = sh;
            sh = sh > 8 ? sh - 8 : 0;
        }
    }
    // ordered compaction: this wave's (greater, equal) counts, then the
    // counts of the waves before it
    unsigned g = 0, e = 0;
    blocks([&](int, const uint32_t* k4) {
        uint64_t G[4], Q[4];
        cmp4_gt(k4, T, G);
        cmp4_ge(k4, T ? T : 1u, Q);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            g += popc(G[v]);
            e += popc(Q[v] & ~G[v]);
        }
    });
    unsigned* x = xch + NW * 4;
    if (lane == 0) {
        x[wid * 2] = g;
        x[wid * 2 + 1] = e;
    }
    __syncthreads();
    int gsum = 0, esum = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        gsum += w < wid ? int(x[w * 2]) : 0;
        esum += w < wid ? int(x[w * 2 + 1]) : 0;
    }
    blocks([&](int u0, const uint32_t* k4) {
        uint64_t G[4], Q[4];
        cmp4_gt(k4, T, G);
        cmp4_ge(k4, T ? T : 1u, Q);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            Q[v] &= ~G[v];
            const int er = esum + int(below(Q[v]));
            const bool gt = k4[v] > T, eq = k4[v] == T && k4[v] != 0u;
            if (gt || (eq && er < need_eq)) sel[gsum + int(below(G[v])) + min(er, need_eq)] = base + 64 * (u0 + v) + lane;
            gsum += popc(G[v]);
            esum += popc(Q[v]);
        }
    });
    __syncthreads();
    return min(K, ks.nvalid);
}

// Select code for n candidates: the keys per lane the select holds in
// registers (4 up to 1024 candidates, 16 up to 4096), or kSelLds when they
// stay in LDS.  One kernel instantiation per code.
constexpr int kSelLds = 32;
__host__ __device__ constexpr int select_width(int n) { return n <= 1024 ? 4 : n <= 4096 ? 16 : kSelLds; }

// Large selects (keys in LDS) first try a threshold from a sample: the
// top r of kSampleKeys regularly spaced keys, r chosen so that about 4 K
// keys lie at or above the r-th (T0).  All keys >= T0 are counted; when
// there are at least K and at most kGatherMax of them, they hold the top K
// (the K-th largest key is >= T0), and an exact select over just those,
// gathered in index order, gives the result.  Otherwise (a skewed sample,
// heavy ties) the full radix select runs.  Either way the result is exact;
// the sample only decides how much work the exact part does.
constexpr int kSampleKeys = 512;
constexpr int kGatherMax = 1024;
constexpr int kSampledWords = kSampleKeys + 2 * kGatherMax + kSampleKeys + 1;

// LDS words a select needs besides keys [n] and sel [K + 1].
__host__ __device__ inline int select_cand_words(int n, int K) {
    (void)K;
    return kRadixWords + (n > 4096 ? kSampledWords : 0);
}

template <int NT, int E>
__device__ int select_top(const uint32_t* keys, int n, int K, int* sel, int* cand, unsigned* tmp,
                          const KeyStats& ks);

// The sampled path above, for n > 4096 keys in LDS with more than K valid.
// Returns the kept count, or -1 (uniformly) when the full select must run;
// leaves the histogram cleared either way.  cand: select_cand_words() words.
template <int NT>
__device__ int sampled_select(const uint32_t* keys, int n, int K, int* sel, int* cand, unsigned* tmp) {
    uint32_t* smp = reinterpret_cast<uint32_t*>(cand) + kRadixWords;    // [kSampleKeys]
    uint32_t* gk = smp + kSampleKeys;                                    // [kGatherMax] gathered keys
    int* gi = reinterpret_cast<int*>(gk + kGatherMax);                  // [kGatherMax] their indices
    int* ssel = gi + kGatherMax;                                         // [kSampleKeys + 1]
    const int tid = threadIdx.x;
    // odd strides keep the lanes' LDS reads on distinct banks
    const int stride = ((n / kSampleKeys) - 1) | 1;
    unsigned nv = 0, kmin = 0xffffffffu, kmax = 0;
    for (int i = tid; i < kSampleKeys; i += NT) {
        const uint32_t k = keys[i * stride];
        smp[i] = k;
        nv += k != 0u;
        kmin = min(kmin, k ? k : 0xffffffffu);
        kmax = max(kmax, k);
    }
    const KeyStats ss = block_key_stats<NT>(nv, kmin, kmax, tmp);
    const int r = max(1, (4 * K + stride - 1) / stride);
    if (r >= kSampleKeys || ss.nvalid <= r) return -1;
    const int nr = select_top<NT, 4>(smp, kSampleKeys, r, ssel, cand, tmp, ss);
    unsigned mn = 0xffffffffu;
    for (int i = tid; i < nr; i += NT) mn = min(mn, smp[ssel[i]]);
    const uint32_t T0 = block_key_stats<NT>(0u, mn, 0u, tmp).kmin;      // the r-th largest sample
    // keys >= T0 over contiguous ranges of at most 63 keys per thread (for
    // the ordered gather; an odd range length keeps the lanes' reads on
    // distinct LDS banks), read eight at a time from clamped indices (no
    // read under a branch); the thread's passing keys are recorded in a bit
    // mask, so the gather visits only those (a few per thread)
    const int per = ((n + NT - 1) / NT) | 1;          // <= 63 for n <= 15872
    if (per > 63) return -1;
    const int i0 = min(n, tid * per), i1 = min(n, i0 + per);
    constexpr int kU = 8;
    uint64_t pass = 0;
    for (int i = i0; i < i1; i += kU) {
        uint32_t k8[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) k8[u] = keys[min(i + u, n - 1)];
#pragma unroll
        for (int u = 0; u < kU; ++u)
            pass |= uint64_t((i + u < i1) && k8[u] >= T0) << (i + u - i0);
    }
    const unsigned c = unsigned(__builtin_popcountll(pass));
    unsigned total;
    unsigned pos = block_excl_scan<NT>(c, tmp + 16, &total);
    if (total < unsigned(K) || total > unsigned(kGatherMax)) return -1;
    unsigned gmin = 0xffffffffu, gmax = 0;
    while (pass) {
        const int j = __builtin_ctzll(pass);
        pass &= pass - 1;
        const uint32_t k = keys[i0 + j];
        gk[pos] = k;
        gi[pos] = i0 + j;
        ++pos;
        gmin = min(gmin, k);
        gmax = max(gmax, k);
    }
    const KeyStats gs = block_key_stats<NT>(c, gmin, gmax, tmp);       // (its barrier orders the gather)
    const int nk = select_top<NT, 4>(gk, int(total), K, sel, cand, tmp, gs);
    int idx[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int i = tid + u * NT;
        idx[u] = i < nk ? gi[sel[i]] : 0;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int i = tid + u * NT;
        if (i < nk) sel[i] = idx[u];
    }
    __syncthreads();
    return nk;
}

// Workgroup-level: top-K of n keys in LDS (loaded by load_keys, which gave
// ks and cleared cand), E = select_width(n).  sel (K + 1 ints) receives the
// kept indices ascending.  cand: select_cand_words() words; tmp: 32 words.
template <int NT, int E>
__device__ int select_top(const uint32_t* keys, int n, int K, int* sel, int* cand, unsigned* tmp,
                          const KeyStats& ks) {
    static_assert(E == 4 || E == 16 || E == kSelLds, "select code");
    uint32_t* hist = reinterpret_cast<uint32_t*>(cand);
    if (K >= n) {
        // every valid key is kept: ordered compaction
        const int per = (n + NT - 1) / NT;
        const int i0 = min(n, int(threadIdx.x) * per), i1 = min(n, i0 + per);
        unsigned c = 0;
        for (int i = i0; i < i1; ++i) c += keys[i] != 0u;
        unsigned total;
        unsigned pos = block_excl_scan<NT>(c, tmp + 16, &total);
        for (int i = i0; i < i1; ++i)
            if (keys[i]) sel[pos++] = i;
        __syncthreads();
        return int(total);
    }
    if constexpr (E == 4) {
        return radix_select<NT, 4>(keys, n, K, sel, hist, tmp, ks);
    } else if constexpr (E == 16) {
        return radix_select<NT, 16>(keys, n, K, sel, hist, tmp, ks);
    } else {
        if (ks.nvalid > K && K <= 2 * NT) {
            const int nk = sampled_select<NT>(keys, n, K, sel, cand, tmp);
            if (nk >= 0) return nk;
        }
        return radix_select<NT, 0>(keys, n, K, sel, hist, tmp, ks);
    }
}


// Select-width code of a kernel whose kept set is not selected but read
// from kept_idx, where an earlier step left it (a reused pruning stage).
constexpr int kGiven = 1;

// Kept set of stage `st` as kept_idx holds it (ascending token starts,
// -1 padded, as a step wrote it): the entries in [0, L), in their order, to
// sel[0..nk), then -1 up to st.keep.  Returns nk; ends with a barrier.
template <int NT>
__device__ int given_kept(const StageDev& st, const int32_t* kept_st, int64_t L, int* sel, unsigned* tmp) {
    const int per = (st.keep + NT - 1) / NT;
    const int i0 = min(st.keep, int(threadIdx.x) * per), i1 = min(st.keep, i0 + per);
    unsigned c = 0;
    for (int i = i0; i < i1; ++i) {
        const int32_t x = kept_st[i];
        c += x >= 0 && x < L;
    }
    unsigned total;
    unsigned pos = block_excl_scan<NT>(c, tmp, &total);
    for (int i = i0; i < i1; ++i) {
        const int32_t x = kept_st[i];
        if (x >= 0 && x < L) sel[pos++] = x;
    }
    for (int i = int(total) + threadIdx.x; i < st.keep; i += NT) sel[i] = -1;
    __syncthreads();
    return int(total);
}

// LDS words kept_of_stage uses: keys [ncand], sel [keep + 1], select
// scratch, and (after the first stage) the parents [ncand / ratio].
__host__ __device__ inline int kept_lds_words(const StageDev& st, bool first_stage) {
    return st.ncand + st.keep + 1 + select_cand_words(st.ncand, st.keep) + (first_stage ? 0 : st.ncand / st.ratio);
}

// Kept set of stage `st` for one (request, KV head), from that stage's
// scores (global, INT32_MIN = no candidate).  Returns nk; the kept chunk
// starts, ascending, are sel[0..nk) with sel = (int*)(lds + st.ncand).
// `parents` are the kept starts of the stage before (global, -1 padded;
// unused for the first stage): they are staged in LDS together with the
// scores, so turning selected indices into starts costs no memory latency
// after the select.  lds: kept_lds_words(st, first_stage) words.
// idx_out (optional, nk words): the kept candidates' indices, ascending.
template <int NT, int E>
__device__ int kept_of_stage(const StageDev& st, bool first_stage, const int32_t* scores_bj,
                             const int32_t* parents, int64_t L, uint32_t* lds, unsigned* tmp, int pslot = -1,
                             int* idx_out = nullptr) {
    (void)pslot;                 // phase-stamp slot (latency studies only)
    uint32_t* keys = lds;
    int* sel = reinterpret_cast<int*>(lds + st.ncand);
    int* cand = sel + st.keep + 1;
    int* par = cand + select_cand_words(st.ncand, st.keep);
    const KeyStats ks = load_keys<NT>(scores_bj, st.ncand, keys, reinterpret_cast<uint32_t*>(cand), tmp, parents,
                                      first_stage ? 0 : st.ncand / st.ratio, par);
    if (pslot >= 0) SD_PHASE(pslot, 6);
    const int nk = select_top<NT, E>(keys, st.ncand, st.keep, sel, cand, tmp, ks);
    if (pslot >= 0) SD_PHASE(pslot, 7);
    for (int i = threadIdx.x; i < nk; i += NT) {
        const int ci = sel[i];
        if (idx_out) idx_out[i] = ci;
        sel[i] = int(cand_start(st, first_stage, par, ci, L));
    }
    __syncthreads();
    return nk;
}

// Fused last two stages P (= S-2) and Q (= S-1), for one (request, KV head):
// select P from its scores, gather the precomputed Q scores of the kept P
// chunks' children, select Q.  LDS words:
//   P select [kept_lds_words(P)] | all children's Q scores [P.ncand * rq] |
//   Q keys [Q.ncand] | Q sel [Q.keep + 1] | Q select scratch | P starts [P.keep]
__host__ __device__ inline int fused_lds_words(const StageDev& P, bool p_first, const StageDev& Q, int rq) {
    return kept_lds_words(P, p_first) + P.ncand * rq + Q.ncand + Q.keep + 1 + select_cand_words(Q.ncand, Q.keep) +
           P.keep;
}

struct FusedOut {
    int* p_starts;      // LDS [P.keep]: P's kept starts, ascending, -1 padded
    int np;             // kept P chunks
    int* q_starts;      // LDS [Q.keep + 1]: Q's kept starts, ascending
    int nq;             // kept Q chunks
    const uint32_t* q_keys;   // LDS [Q.ncand]: Q's candidate keys
};

template <int NT, int EP, int EQ>
__device__ FusedOut kept_two_stages(const StageDev& P, bool p_first, const int32_t* scoresP_bj,
                                    const int32_t* parentsP, const int32_t* pre_bj, int rq, const StageDev& Q,
                                    int64_t L, uint32_t* lds, unsigned* tmp) {
    uint32_t* keysP = lds;
    int* selP = reinterpret_cast<int*>(lds + P.ncand);
    int* candP = selP + P.keep + 1;
    int* parP = candP + select_cand_words(P.ncand, P.keep);
    int* preL = parP + (p_first ? 0 : P.ncand / P.ratio);
    uint32_t* keysQ = reinterpret_cast<uint32_t*>(preL + P.ncand * rq);
    int* selQ = reinterpret_cast<int*>(keysQ + Q.ncand);
    int* candQ = selQ + Q.keep + 1;
    int* startsP = candQ + select_cand_words(Q.ncand, Q.keep);

    // the first batch of the children's Q scores is issued, then P's parents
    // and scores (load_keys): one memory round trip for all of them up to
    // kLoadBatch * NT children (the loads of a wave complete in issue order)
    const int npre = P.ncand * rq;
    int32_t v0[kLoadBatch];
#pragma unroll
    for (int u = 0; u < kLoadBatch; ++u) {
        const int i = threadIdx.x + u * NT;
        v0[u] = i < npre ? pre_bj[i] : 0;
    }
    const KeyStats ksP = load_keys<NT>(scoresP_bj, P.ncand, keysP, reinterpret_cast<uint32_t*>(candP), tmp, parentsP,
                                       p_first ? 0 : P.ncand / P.ratio, parP);
#pragma unroll
    for (int u = 0; u < kLoadBatch; ++u)
        if (threadIdx.x + u * NT < npre) preL[threadIdx.x + u * NT] = v0[u];
    for (int i0 = threadIdx.x + kLoadBatch * NT; i0 < npre; i0 += kLoadBatch * NT) {
        int32_t v[kLoadBatch];
#pragma unroll
        for (int u = 0; u < kLoadBatch; ++u) {
            const int i = i0 + u * NT;
            v[u] = i < npre ? pre_bj[i] : 0;
        }
#pragma unroll
        for (int u = 0; u < kLoadBatch; ++u)
            if (i0 + u * NT < npre) preL[i0 + u * NT] = v[u];
    }
    SD_PHASE(3, 8);
    const int np = select_top<NT, EP>(keysP, P.ncand, P.keep, selP, candP, tmp, ksP);
    SD_PHASE(3, 9);
    // P starts; Q candidate i is child i % rq of kept P chunk i / rq
    for (int i = threadIdx.x; i < P.keep; i += NT)
        startsP[i] = i < np ? int(cand_start(P, p_first, parP, selP[i], L)) : -1;
    SD_PHASE(3, 12);
    if (threadIdx.x < 256) candQ[threadIdx.x] = 0;
    unsigned nv = 0, kmin = 0xffffffffu, kmax = 0;
    for (int i = threadIdx.x; i < Q.ncand; i += NT) {
        const int q = i / rq;
        const uint32_t k = q < np ? score_key(preL[selP[q] * rq + (i - q * rq)]) : 0u;
        keysQ[i] = k;
        nv += k != 0u;
        kmin = min(kmin, k ? k : 0xffffffffu);
        kmax = max(kmax, k);
    }
    SD_PHASE(3, 13);
    const KeyStats ksQ = block_key_stats<NT>(nv, kmin, kmax, tmp);
    SD_PHASE(3, 10);
    const int nq = select_top<NT, EQ>(keysQ, Q.ncand, Q.keep, selQ, candQ, tmp, ksQ);
    SD_PHASE(3, 11);
    for (int i = threadIdx.x; i < nq; i += NT) {
        const int c = selQ[i], q = c / rq;
        selQ[i] = startsP[q] + (c - q * rq) * Q.chunk;
    }
    __syncthreads();
    return FusedOut{startsP, np, selQ, nq, keysQ};
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
    auto first_block = [&](int c) -> int64_t { return int64_t(kept_s[c]) >> 3; };
    // first kept chunk whose last block is >= v (nk if none): a search over
    // the chunks, with no division in its loop
    auto chunk_lower = [&](int64_t v) -> int {
        int lo = 0, hi = nk;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (first_block(mid) + bpc - 1 < v) lo = mid + 1; else hi = mid;
        }
        return lo;
    };
    auto lower = [&](int64_t v) -> int {     // first q with blk_at(q) >= v
        const int c = chunk_lower(v);
        if (c >= nk) return nq;
        const int64_t off = v - first_block(c);
        return c * bpc + int(off > 0 ? off : 0);
    };
    auto kept_block = [&](int64_t blk) -> bool {
        const int c = chunk_lower(blk);
        return c < nk && first_block(c) <= blk;
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
