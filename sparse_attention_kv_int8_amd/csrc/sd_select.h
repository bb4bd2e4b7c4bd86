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

// Keys the cooperative select of a 256-thread workgroup holds in registers
// (16 per lane); more stay in LDS (coop_select_lds).
constexpr int kSelRegMax = 4096;
// Undecided keys coop_select_lds moves from LDS to registers (4 per lane).
constexpr int kSelList = 1024;

// LDS words the select needs besides keys [n] and sel [K + 1] (the
// cooperative selects exchange their counts through the workgroup's 32-word
// scratch): the list of undecided keys of coop_select_lds.
__host__ __device__ inline int select_cand_words(int n, int K) {
    return n > kSelRegMax && K < n ? kSelList : 0;
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
// larger key is better and equal keys go to the lower index.  One wave
// finds the threshold T (the K-th largest key) two bits per round, counting
// with compares into scalar masks and scalar popcounts, then compacts the
// kept positions in order: no barrier, no LDS atomics and no cross-lane
// reduction chain inside the search.
// ------------------------------------------------------------------------
constexpr int kKeyBits = 24;

__device__ __forceinline__ uint32_t score_key(int s) {
    return s == INT32_MIN ? 0u : uint32_t(s + (1 << 23));
}

// Compares of 4 keys against wave-uniform thresholds, each into its own
// scalar register pair (the lanes that pass), issued back to back: a
// compare's mask is ready for its scalar popcount only some 30 cycles
// later, so the compares of a block overlap that latency.
#define SD_CMP(op, d, v, t) "v_cmp_" op "_u32_e64 %" #d ", %" #v ", %" #t "\n\t"
__device__ __forceinline__ void cmp4x3_ge(const uint32_t* k, uint32_t t1, uint32_t t2, uint32_t t3, uint64_t* m) {
    asm(SD_CMP("ge", 0, 12, 16) SD_CMP("ge", 1, 12, 17) SD_CMP("ge", 2, 12, 18)
        SD_CMP("ge", 3, 13, 16) SD_CMP("ge", 4, 13, 17) SD_CMP("ge", 5, 13, 18)
        SD_CMP("ge", 6, 14, 16) SD_CMP("ge", 7, 14, 17) SD_CMP("ge", 8, 14, 18)
        SD_CMP("ge", 9, 15, 16) SD_CMP("ge", 10, 15, 17) SD_CMP("ge", 11, 15, 18)
        : "=&s"(m[0]), "=&s"(m[1]), "=&s"(m[2]), "=&s"(m[3]), "=&s"(m[4]), "=&s"(m[5]),
          "=&s"(m[6]), "=&s"(m[7]), "=&s"(m[8]), "=&s"(m[9]), "=&s"(m[10]), "=&s"(m[11])
        : "v"(k[0]), "v"(k[1]), "v"(k[2]), "v"(k[3]), "s"(__builtin_amdgcn_readfirstlane(t1)),
          "s"(__builtin_amdgcn_readfirstlane(t2)), "s"(__builtin_amdgcn_readfirstlane(t3)));
}
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

// Sign bit of a wave-uniform value as 0/1 in a scalar register (written out
// because the compiler turns the equivalent comparison into a round trip
// through a vector register).
__device__ __forceinline__ int sign_bit_s(int v) {
    int r;
    asm("s_lshr_b32 %0, %1, 31" : "=s"(r) : "s"(__builtin_amdgcn_readfirstlane(v)));
    return r;
}

// One full wave: top-K of m keys key(i) = keys[idx ? idx[i] : i], m <= 64 E
// <= 1024.  Slot u of lane l holds position i = 64 u + l (conflict-free LDS
// reads; ascending i is slot-major).  Writes the kept positions i, ascending,
// to out[0..kept) (out has K + 1 slots); returns kept = min(K, #valid).
//
// The threshold T (the K-th largest key) is built two bits per round from
// the top: the counts of keys >= prefix + {1,2,3} << b come from compares
// into scalar masks and scalar popcounts, and the largest threshold whose
// count reaches K extends the prefix.  The search stops early once exactly K
// keys lie at or above the prefix (then those are the top K and no tie needs
// breaking).  Keys > T are kept, and of the keys equal to T the lowest
// positions, K - #(keys > T) of them.
template <int E>
__device__ __forceinline__ int wave_select_e(const uint32_t* keys, const int* idx, int m, int K, int* out) {
    constexpr int EP = E < 4 ? 4 : E;          // slots, padded with empty keys to blocks of 4
    const int lane = threadIdx.x & 63;
    uint32_t kk[EP];
#pragma unroll
    for (int u = 0; u < EP; ++u) {
        const int i = 64 * u + lane;
        kk[u] = (u < E && i < m) ? keys[idx ? idx[i] : i] : 0u;
    }
    int nvalid = 0;
#pragma unroll
    for (int u = 0; u < EP; u += 4) {
        uint64_t mk[4];
        cmp4_ge(kk + u, 1u, mk);
        nvalid += popc(mk[0]) + popc(mk[1]) + popc(mk[2]) + popc(mk[3]);
    }
    uint32_t T = 0;
    int need_eq = 0;
    if (nvalid > K) {
        // Rebase valid keys to key - min + 1 (order and validity kept) so the
        // search starts at the highest bit in which they can differ.
        uint32_t kmin = 0xffffffffu, kmax = 0;
#pragma unroll
        for (int u = 0; u < E; ++u) {
            kmin = min(kmin, kk[u] ? kk[u] : 0xffffffffu);
            kmax = max(kmax, kk[u]);
        }
        kmin = wave_min_u(kmin);
        kmax = wave_max_u(kmax);
#pragma unroll
        for (int u = 0; u < E; ++u) kk[u] = kk[u] ? kk[u] - kmin + 1u : 0u;
        const uint32_t range = kmax - kmin + 1u;              // largest rebased key
        const int bits = 32 - __builtin_clz(range);           // range < 2^bits
        uint32_t prefix = 0;
        int cnt = nvalid;                      // valid keys >= prefix
        bool exact = false;
        // b even with 4 << b > range
        for (int b = bits > 2 ? ((bits - 1) & ~1) : 0; b >= 0; b -= 2) {
            const uint32_t t1 = prefix + (1u << b), t2 = prefix + (2u << b), t3 = prefix + (3u << b);
            int n1 = 0, n2 = 0, n3 = 0;
#pragma unroll
            for (int u = 0; u < EP; u += 4) {
                uint64_t c[12];
                cmp4x3_ge(kk + u, t1, t2, t3, c);
                n1 += popc(c[0]) + popc(c[3]) + popc(c[6]) + popc(c[9]);
                n2 += popc(c[1]) + popc(c[4]) + popc(c[7]) + popc(c[10]);
                n3 += popc(c[2]) + popc(c[5]) + popc(c[8]) + popc(c[11]);
            }
            // n1 >= n2 >= n3: the largest threshold still reaching K is the
            // number of counts >= K (sign bits: n >= K  <=>  K - 1 - n < 0)
            const int c = sign_bit_s(K - 1 - n1) + sign_bit_s(K - 1 - n2) + sign_bit_s(K - 1 - n3);
            prefix += uint32_t(c) << b;
            const int nc = c >= 3 ? n3 : c >= 2 ? n2 : n1;
            cnt = c > 0 ? nc : cnt;
            if (cnt == K) {                    // exactly K keys >= prefix: they are the top K
                exact = true;
                break;
            }
        }
        if (exact) {
            T = prefix - 1u;                   // keys > T are kept, no tie to break
        } else {
            T = prefix;                        // the K-th largest (rebased) key
            int ngt = 0;
#pragma unroll
            for (int u = 0; u < EP; u += 4) {
                uint64_t mk[4];
                cmp4_gt(kk + u, T, mk);
                ngt += popc(mk[0]) + popc(mk[1]) + popc(mk[2]) + popc(mk[3]);
            }
            need_eq = K - ngt;
        }
    }
    // ordered compaction: a kept key goes to #(greater keys before it) +
    // min(#(equal keys before it), need_eq); "before" = smaller position.
    // Masks are taken four slots at a time (few scalar registers live).
    int gsum = 0, esum = 0;
#pragma unroll
    for (int u0 = 0; u0 < EP; u0 += 4) {
        uint64_t G[4];
        cmp4_gt(kk + u0, T, G);
        if (need_eq == 0) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int u = u0 + v;
                if (u < E && kk[u] > T) out[gsum + int(below(G[v]))] = 64 * u + lane;
                gsum += popc(G[v]);
            }
        } else {
            // equal keys: >= T and not > T (T >= 1 here, so they are valid keys)
            uint64_t Q[4];
            cmp4_ge(kk + u0, T, Q);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int u = u0 + v;
                Q[v] &= ~G[v];
                const int er = esum + int(below(Q[v]));
                const bool gt = kk[u] > T, eq = kk[u] == T;
                if (u < E && (gt || (eq && er < need_eq))) out[gsum + int(below(G[v])) + min(er, need_eq)] = 64 * u + lane;
                gsum += popc(G[v]);
                esum += popc(Q[v]);
            }
        }
    }
    return min(K, nvalid);
}

// All NW waves of the workgroup together: top-K of n <= NW * 64 * EW keys
// in LDS.  Wave w holds positions [w * 64 EW, (w + 1) * 64 EW) (slot-major,
// so ascending position is wave-major), counts its own keys against each
// round's thresholds, and the per-wave counts are added through LDS (xch:
// 2 x NW x 4 words, double buffered, so one barrier per round).  Every wave
// takes the same decisions from the same totals.  Writes the kept positions,
// ascending, to sel; ends with a barrier; returns min(K, #valid).
template <int NT, int EW>
__device__ int coop_select(const uint32_t* keys, int n, int K, int* sel, unsigned* xch) {
    constexpr int NW = NT / kWave;
    static_assert(EW % 4 == 0 && 2 * NW * 4 <= 32, "coop_select layout");
    const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int base = wid * 64 * EW;
    uint32_t kk[EW];
#pragma unroll
    for (int u = 0; u < EW; ++u) {
        const int i = base + 64 * u + lane;
        kk[u] = i < n ? keys[i] : 0u;
    }
    int nv = 0;
    uint32_t kmin = 0xffffffffu, kmax = 0;
#pragma unroll
    for (int u = 0; u < EW; u += 4) {
        uint64_t mk[4];
        cmp4_ge(kk + u, 1u, mk);
        nv += popc(mk[0]) + popc(mk[1]) + popc(mk[2]) + popc(mk[3]);
    }
#pragma unroll
    for (int u = 0; u < EW; ++u) {
        kmin = min(kmin, kk[u] ? kk[u] : 0xffffffffu);
        kmax = max(kmax, kk[u]);
    }
    kmin = wave_min_u(kmin);
    kmax = wave_max_u(kmax);
    int buf = 0;
    auto exchange3 = [&](unsigned a, unsigned b, unsigned c, unsigned (&tot)[3], unsigned* before) {
        unsigned* x = xch + buf * (NW * 4);
        if (lane == 0) {
            x[wid * 4] = a;
            x[wid * 4 + 1] = b;
            x[wid * 4 + 2] = c;
        }
        __syncthreads();
        tot[0] = tot[1] = tot[2] = 0;
        if (before) before[0] = before[1] = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const unsigned xa = x[w * 4], xb = x[w * 4 + 1], xc = x[w * 4 + 2];
            if (before && w < wid) { before[0] += xa; before[1] += xb; }
            tot[0] += xa;
            tot[1] += xb;
            tot[2] += xc;
        }
        buf ^= 1;
    };
    // valid count; min and max travel as a sum-free pair (min of mins via
    // ~max of complements)
    unsigned t0[3];
    {
        unsigned* x = xch + buf * (NW * 4);
        if (lane == 0) {
            x[wid * 4] = unsigned(nv);
            x[wid * 4 + 1] = kmin;
            x[wid * 4 + 2] = kmax;
        }
        __syncthreads();
        t0[0] = 0;
        t0[1] = 0xffffffffu;
        t0[2] = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            t0[0] += x[w * 4];
            t0[1] = min(t0[1], x[w * 4 + 1]);
            t0[2] = max(t0[2], x[w * 4 + 2]);
        }
        buf ^= 1;
    }
    const int nvalid = int(t0[0]);
    uint32_t T = 0;
    int need_eq = 0;
    if (nvalid > K) {
        const uint32_t gmin = t0[1], gmax = t0[2];
#pragma unroll
        for (int u = 0; u < EW; ++u) kk[u] = kk[u] ? kk[u] - gmin + 1u : 0u;
        const uint32_t range = gmax - gmin + 1u;
        const int bits = 32 - __builtin_clz(range);
        uint32_t prefix = 0;
        int cnt = nvalid;
        bool exact = false;
        for (int b = bits > 2 ? ((bits - 1) & ~1) : 0; b >= 0; b -= 2) {
            const uint32_t t1 = prefix + (1u << b), t2 = prefix + (2u << b), t3 = prefix + (3u << b);
            unsigned n1 = 0, n2 = 0, n3 = 0;
#pragma unroll
            for (int u = 0; u < EW; u += 4) {
                uint64_t c[12];
                cmp4x3_ge(kk + u, t1, t2, t3, c);
                n1 += popc(c[0]) + popc(c[3]) + popc(c[6]) + popc(c[9]);
                n2 += popc(c[1]) + popc(c[4]) + popc(c[7]) + popc(c[10]);
                n3 += popc(c[2]) + popc(c[5]) + popc(c[8]) + popc(c[11]);
            }
            unsigned tot[3];
            exchange3(n1, n2, n3, tot, nullptr);
            const int N1 = int(tot[0]), N2 = int(tot[1]), N3 = int(tot[2]);
            const int c = sign_bit_s(K - 1 - N1) + sign_bit_s(K - 1 - N2) + sign_bit_s(K - 1 - N3);
            prefix += uint32_t(c) << b;
            const int nc = c >= 3 ? N3 : c >= 2 ? N2 : N1;
            cnt = c > 0 ? nc : cnt;
            if (cnt == K) {
                exact = true;
                break;
            }
        }
        if (exact) {
            T = prefix - 1u;
        } else {
            T = prefix;
            unsigned ng = 0;
#pragma unroll
            for (int u = 0; u < EW; u += 4) {
                uint64_t mk[4];
                cmp4_gt(kk + u, T, mk);
                ng += popc(mk[0]) + popc(mk[1]) + popc(mk[2]) + popc(mk[3]);
            }
            unsigned tot[3];
            exchange3(ng, 0u, 0u, tot, nullptr);
            need_eq = K - int(tot[0]);
        }
    }
    // ordered compaction: this wave's (greater, equal) counts, then the
    // counts of the waves before it
    unsigned g = 0, e = 0;
#pragma unroll
    for (int u = 0; u < EW; u += 4) {
        uint64_t G[4], Q[4];
        cmp4_gt(kk + u, T, G);
        cmp4_ge(kk + u, T ? T : 1u, Q);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            g += popc(G[v]);
            e += popc(Q[v] & ~G[v]);
        }
    }
    unsigned tot[3], before[2];
    exchange3(g, e, 0u, tot, before);
    int gsum = int(before[0]), esum = int(before[1]);
#pragma unroll
    for (int u0 = 0; u0 < EW; u0 += 4) {
        uint64_t G[4];
        cmp4_gt(kk + u0, T, G);
        if (need_eq == 0) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int u = u0 + v;
                if (kk[u] > T) sel[gsum + int(below(G[v]))] = base + 64 * u + lane;
                gsum += popc(G[v]);
            }
        } else {
            uint64_t Q[4];
            cmp4_ge(kk + u0, T, Q);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int u = u0 + v;
                Q[v] &= ~G[v];
                const int er = esum + int(below(Q[v]));
                const bool gt = kk[u] > T, eq = kk[u] == T;
                if (gt || (eq && er < need_eq)) sel[gsum + int(below(G[v])) + min(er, need_eq)] = base + 64 * u + lane;
                gsum += popc(G[v]);
                esum += popc(Q[v]);
            }
        }
    }
    __syncthreads();
    return min(K, nvalid);
}

// coop_select for more keys than the waves hold in registers: the keys stay
// in LDS, and each wave reads its share in blocks of 4 slots per pass (the
// loop over blocks is not unrolled, which bounds register use).  The 2-bit
// rounds leave undecided only the keys whose bits above the current digit
// equal the prefix found so far; once those are at most kSelList, they are
// copied to `lst` (LDS) and the remaining rounds count them from registers,
// 4 per lane, adding the count above that bucket.  The final compaction
// reads every key again.  Full passes: min/max, the rounds before the copy
// (one or two on spread-out scores), the copy, and two for the compaction.

template <int NT>
__device__ int coop_select_lds(const uint32_t* keys, int n, int K, int* sel, unsigned* xch, uint32_t* lst) {
    constexpr int NW = NT / kWave;
    static_assert(NW * kWave * 4 == kSelList, "the list is held 4 keys per lane");
    const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int per_wave = (n + NW - 1) / NW;
    const int nblk = ((per_wave + 63) / 64 + 3) / 4;        // blocks of 4 slots per wave
    const int base = wid * nblk * 4 * 64;
    auto key_at = [&](int u) -> uint32_t {
        const int i = base + 64 * u + lane;
        return i < n ? keys[i] : 0u;
    };
    int buf = 0;
    // totals over the waves of (a, b, c) (or min of b and max of c), and
    // the sums of a and b over the waves before this one
    auto exchange = [&](unsigned a, unsigned b, unsigned c, unsigned (&tot)[3], unsigned* before, bool minmax) {
        unsigned* x = xch + buf * (NW * 4);
        if (lane == 0) {
            x[wid * 4] = a;
            x[wid * 4 + 1] = b;
            x[wid * 4 + 2] = c;
        }
        __syncthreads();
        tot[0] = 0;
        tot[1] = minmax ? 0xffffffffu : 0u;
        tot[2] = 0;
        if (before) before[0] = before[1] = 0;
        for (int w = 0; w < NW; ++w) {
            const unsigned xa = x[w * 4], xb = x[w * 4 + 1], xc = x[w * 4 + 2];
            if (before && w < wid) {
                before[0] += xa;
                before[1] += xb;
            }
            tot[0] += xa;
            tot[1] = minmax ? min(tot[1], xb) : tot[1] + xb;
            tot[2] = minmax ? max(tot[2], xc) : tot[2] + xc;
        }
        buf ^= 1;
    };
    unsigned nv = 0, kmin = 0xffffffffu, kmax = 0;
#pragma unroll 1
    for (int u0 = 0; u0 < nblk * 4; u0 += 4) {
        uint32_t k4[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            k4[v] = key_at(u0 + v);
            kmin = min(kmin, k4[v] ? k4[v] : 0xffffffffu);
            kmax = max(kmax, k4[v]);
        }
        uint64_t mk[4];
        cmp4_ge(k4, 1u, mk);
        nv += popc(mk[0]) + popc(mk[1]) + popc(mk[2]) + popc(mk[3]);
    }
    kmin = wave_min_u(kmin);
    kmax = wave_max_u(kmax);
    unsigned t0[3];
    exchange(nv, kmin, kmax, t0, nullptr, true);
    const int nvalid = int(t0[0]);
    const uint32_t gmin = t0[1];
    auto rk = [&](uint32_t k) -> uint32_t { return k ? k - gmin + 1u : 0u; };   // rebased, order and validity kept
    uint32_t T = 0;
    int need_eq = 0;
    if (nvalid > K) {
        const uint32_t range = t0[2] - gmin + 1u;
        const int bits = 32 - __builtin_clz(range);
        uint32_t prefix = 0;
        int cnt = nvalid;        // valid keys >= prefix
        int above = 0;           // keys >= prefix + (1 << b) after a round at b
        int cnt_w = int(nv), above_w = 0;                    // the same, this wave's keys (before the copy)
        bool listed = false;
        int above0 = 0;          // keys above the copied bucket
        uint32_t lk[4] = {0u, 0u, 0u, 0u};
        bool exact = false;
        for (int b = bits > 2 ? ((bits - 1) & ~1) : 0; b >= 0; b -= 2) {
            const uint32_t t1 = prefix + (1u << b), t2 = prefix + (2u << b), t3 = prefix + (3u << b);
            unsigned n1 = 0, n2 = 0, n3 = 0;
            if (listed) {
                uint64_t c[12];
                cmp4x3_ge(lk, t1, t2, t3, c);
                n1 = popc(c[0]) + popc(c[3]) + popc(c[6]) + popc(c[9]);
                n2 = popc(c[1]) + popc(c[4]) + popc(c[7]) + popc(c[10]);
                n3 = popc(c[2]) + popc(c[5]) + popc(c[8]) + popc(c[11]);
            } else {
#pragma unroll 1
                for (int u0 = 0; u0 < nblk * 4; u0 += 4) {
                    uint32_t k4[4];
#pragma unroll
                    for (int v = 0; v < 4; ++v) k4[v] = rk(key_at(u0 + v));
                    uint64_t c[12];
                    cmp4x3_ge(k4, t1, t2, t3, c);
                    n1 += popc(c[0]) + popc(c[3]) + popc(c[6]) + popc(c[9]);
                    n2 += popc(c[1]) + popc(c[4]) + popc(c[7]) + popc(c[10]);
                    n3 += popc(c[2]) + popc(c[5]) + popc(c[8]) + popc(c[11]);
                }
            }
            unsigned tot[3];
            exchange(n1, n2, n3, tot, nullptr, false);
            const int N1 = int(tot[0]) + above0, N2 = int(tot[1]) + above0, N3 = int(tot[2]) + above0;
            const int c = sign_bit_s(K - 1 - N1) + sign_bit_s(K - 1 - N2) + sign_bit_s(K - 1 - N3);
            prefix += uint32_t(c) << b;
            if (c > 0) {
                cnt = c >= 3 ? N3 : c >= 2 ? N2 : N1;
                cnt_w = int(c >= 3 ? n3 : c >= 2 ? n2 : n1);
            }
            if (c < 3) {
                above = c >= 2 ? N3 : c >= 1 ? N2 : N1;
                above_w = int(c >= 2 ? n3 : c >= 1 ? n2 : n1);
            }
            if (cnt == K) {
                exact = true;
                break;
            }
            if (!listed && b >= 2 && cnt - above <= kSelList) {
                // copy the undecided bucket [max(prefix, 1), prefix + (1 << b)) to lst
                unsigned tw[3], bw[2];
                exchange(unsigned(cnt_w - above_w), 0u, 0u, tw, bw, false);
                const uint32_t lo = prefix ? prefix : 1u, hi = prefix + (1u << b);
                int pos = int(bw[0]);
#pragma unroll 1
                for (int u0 = 0; u0 < nblk * 4; u0 += 4) {
                    uint32_t k4[4];
#pragma unroll
                    for (int v = 0; v < 4; ++v) k4[v] = rk(key_at(u0 + v));
                    uint64_t A[4], B[4];
                    cmp4_ge(k4, lo, A);
                    cmp4_ge(k4, hi, B);
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const uint64_t in = A[v] & ~B[v];
                        if (k4[v] >= lo && k4[v] < hi) lst[pos + int(below(in))] = k4[v];
                        pos += popc(in);
                    }
                }
                __syncthreads();
                const int U = int(tw[0]);
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int i = wid * 256 + 64 * v + lane;
                    lk[v] = i < U ? lst[i] : 0u;
                }
                above0 = above;
                listed = true;
            }
        }
        if (exact) {
            T = prefix - 1u;
        } else {
            T = prefix;
            unsigned ng = 0;
            if (listed) {
                uint64_t mk[4];
                cmp4_gt(lk, T, mk);
                ng = popc(mk[0]) + popc(mk[1]) + popc(mk[2]) + popc(mk[3]);
            } else {
#pragma unroll 1
                for (int u0 = 0; u0 < nblk * 4; u0 += 4) {
                    uint32_t k4[4];
#pragma unroll
                    for (int v = 0; v < 4; ++v) k4[v] = rk(key_at(u0 + v));
                    uint64_t mk[4];
                    cmp4_gt(k4, T, mk);
                    ng += popc(mk[0]) + popc(mk[1]) + popc(mk[2]) + popc(mk[3]);
                }
            }
            unsigned tot[3];
            exchange(ng, 0u, 0u, tot, nullptr, false);
            need_eq = K - (int(tot[0]) + above0);
        }
    }
    // ordered compaction (positions are wave-major, then slot-major)
    unsigned g = 0, e = 0;
#pragma unroll 1
    for (int u0 = 0; u0 < nblk * 4; u0 += 4) {
        uint32_t k4[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) k4[v] = rk(key_at(u0 + v));
        uint64_t G[4], Q[4];
        cmp4_gt(k4, T, G);
        cmp4_ge(k4, T ? T : 1u, Q);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            g += popc(G[v]);
            e += popc(Q[v] & ~G[v]);
        }
    }
    unsigned tot[3], before[2];
    exchange(g, e, 0u, tot, before, false);
    int gsum = int(before[0]), esum = int(before[1]);
#pragma unroll 1
    for (int u0 = 0; u0 < nblk * 4; u0 += 4) {
        uint32_t k4[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) k4[v] = rk(key_at(u0 + v));
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
    }
    __syncthreads();
    return min(K, nvalid);
}

// Select width for n candidates: 8 keys per lane of one wave up to 512, else
// 16 (the cooperative selects of select_top).
__host__ __device__ constexpr int select_width(int n) { return n <= 512 ? 8 : 16; }

// Block-level: top-K of n keys in LDS, with E = select_width(n): up to 512
// keys one wave selects alone (8 per lane); more are split between the
// waves, which search the threshold together, holding 4 or 16 keys per lane
// in registers (coop_select) or, past NW * 1024 keys, reading them from LDS
// in every pass (coop_select_lds).  sel (K + 1 ints) receives the kept indices ascending.
// cand: select_cand_words(n, K) words of LDS.  tmp: 32 words of LDS.
template <int NT, int E>
__device__ int select_top(const uint32_t* keys, int n, int K, int* sel, int* cand, unsigned* tmp) {
    static_assert(E == 8 || E == 16, "select width");
    static_assert(E == 8 || NT * 16 == kSelRegMax, "the cooperative select is laid out for 256 threads");
    constexpr int NW = NT / kWave;
    const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
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
    } else if (E == 16 && n <= NW * 64 * 4) {
        kept = coop_select<NT, 4>(keys, n, K, sel, tmp);
    } else if (E == 16 && n <= NW * 64 * 16) {
        kept = coop_select<NT, 16>(keys, n, K, sel, tmp);
    } else if (E == 16) {
        kept = coop_select_lds<NT>(keys, n, K, sel, tmp, reinterpret_cast<uint32_t*>(cand));
    } else {                                                  // width 8: n <= 512, one wave
        if (wid == 0) {
            const int r = wave_select_e<E>(keys, nullptr, n, K, sel);
            if (lane == 0) tmp[0] = unsigned(r);
        }
        __syncthreads();
        kept = int(tmp[0]);
    }
    return kept;
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
template <int NT, int E>
__device__ int kept_of_stage(const StageDev& st, bool first_stage, const int32_t* scores_bj,
                             const int32_t* parents, int64_t L, uint32_t* lds, unsigned* tmp) {
    uint32_t* keys = lds;
    int* sel = reinterpret_cast<int*>(lds + st.ncand);
    int* cand = sel + st.keep + 1;
    int* par = cand + select_cand_words(st.ncand, st.keep);
    for (int i = threadIdx.x; i < st.ncand; i += NT) keys[i] = score_key(scores_bj[i]);
    if (!first_stage)
        for (int i = threadIdx.x; i < st.ncand / st.ratio; i += NT) par[i] = parents[i];
    __syncthreads();
    const int nk = select_top<NT, E>(keys, st.ncand, st.keep, sel, cand, tmp);
    for (int i = threadIdx.x; i < nk; i += NT) sel[i] = int(cand_start(st, first_stage, par, sel[i], L));
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

    // every load is issued up front: P's scores, P's parents, all children's Q scores
    for (int i = threadIdx.x; i < P.ncand; i += NT) keysP[i] = score_key(scoresP_bj[i]);
    if (!p_first)
        for (int i = threadIdx.x; i < P.ncand / P.ratio; i += NT) parP[i] = parentsP[i];
    for (int i = threadIdx.x; i < P.ncand * rq; i += NT) preL[i] = pre_bj[i];
    __syncthreads();
    const int np = select_top<NT, EP>(keysP, P.ncand, P.keep, selP, candP, tmp);
    // P starts; Q candidate i is child i % rq of kept P chunk i / rq
    for (int i = threadIdx.x; i < P.keep; i += NT)
        startsP[i] = i < np ? int(cand_start(P, p_first, parP, selP[i], L)) : -1;
    for (int i = threadIdx.x; i < Q.ncand; i += NT) {
        const int q = i / rq;
        keysQ[i] = q < np ? score_key(preL[selP[q] * rq + (i - q * rq)]) : 0u;
    }
    __syncthreads();
    const int nq = select_top<NT, EQ>(keysQ, Q.ncand, Q.keep, selQ, candQ, tmp);
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
