// Device helpers shared by the sparse decode kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sd {

// Phase timestamps for latency studies, compiled in only with
// -DSD_PHASE_STAMPS: thread 0 of each workgroup records the 100 MHz
// s_memrealtime counter at the marked points of a kernel, into
// buf[slot][linear workgroup][phase], with buf set per source file by its
// sd_phase_setup_* function.
#ifdef SD_PHASE_STAMPS
static __device__ unsigned long long* g_phase_buf;
static __device__ int g_phase_maxwg;
__device__ __forceinline__ void phase_stamp(int slot, int phase) {
    unsigned long long* buf = g_phase_buf;
    const int g = int(blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z));
    if (buf && threadIdx.x == 0 && g < g_phase_maxwg)
        buf[(int64_t(slot) * g_phase_maxwg + g) * 16 + phase] = __builtin_amdgcn_s_memrealtime();
}
#define SD_PHASE(slot, phase) ::sd::phase_stamp((slot), (phase))
#define SD_PHASE_SETUP(name)                                                                            \
    extern "C" int sd_phase_setup_##name(unsigned long long* buf, int maxwg) {                          \
        if (hipMemcpyToSymbol(HIP_SYMBOL(::sd::g_phase_buf), &buf, sizeof(buf)) != hipSuccess) return 1; \
        return hipMemcpyToSymbol(HIP_SYMBOL(::sd::g_phase_maxwg), &maxwg, sizeof(int)) != hipSuccess;   \
    }
#else
#define SD_PHASE(slot, phase) ((void)0)
#define SD_PHASE_SETUP(name)
#endif

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kHeadDim = 128;

// ---------------------------------------------------------------- bf16 ----
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// fp32 -> bf16, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return uint16_t(u >> 16);
}

// Symmetric int8 code of one bf16 value: rint((127 * x) / scale).
// 127 * x is exact in fp32 (bf16 carries 8 significant bits) and the
// division is correctly rounded (the library is built with
// -fhip-fp32-correctly-rounded-divide-sqrt), so the code equals the exact
// rational round-half-even.  scale == 0 gives 0.
__device__ __forceinline__ int code_of(float x, float scale) {
    if (scale == 0.0f) return 0;
    return int(__builtin_rintf((127.0f * x) / scale));
}

// Symmetric 4-bit code of one bf16 value: rint((7 * x) / scale) in
// [-7, 7] (7 * x is exact in fp32, the division correctly rounded, as
// above).  scale == 0 gives 0.
__device__ __forceinline__ int code4_of(float x, float scale) {
    if (scale == 0.0f) return 0;
    return int(__builtin_rintf((7.0f * x) / scale));
}

// ----------------------------------------------------------- DPP moves ----
// quad_perm [1,0,3,2] (lane ^ 1), quad_perm [2,3,0,1] (lane ^ 2),
// row_half_mirror (lane i <-> 7 - i inside each group of 8),
// row_ror:8 (lane ^ 8 inside each row of 16).
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;
constexpr int kDppXor2 = 0x4E;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppRor8 = 0x128;

// Sum over the 8 consecutive lanes 8g..8g+7; every lane of the group gets it.
__device__ __forceinline__ int sum8_i(int v) {
    v += dpp_i<kDppXor1>(v);
    v += dpp_i<kDppXor2>(v);
    v += dpp_i<kDppHalfMirror>(v);
    return v;
}
__device__ __forceinline__ float sum8_f(float v) {
    v += dpp_f<kDppXor1>(v);
    v += dpp_f<kDppXor2>(v);
    v += dpp_f<kDppHalfMirror>(v);
    return v;
}

// Max / sum across the 8 lane groups of a wave (lanes differing in bits
// 3..5), for values that are equal inside each group of 8: row_ror:8 pairs
// the two groups of a row, readlane combines the four rows.  The result is
// wave-uniform.
__device__ __forceinline__ int max_groups_i(int v) {
    v = max(v, dpp_i<kDppRor8>(v));
    return max(max(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
               max(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}
__device__ __forceinline__ float rl_f(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}
__device__ __forceinline__ float max_groups_f(float v) {
    v = fmaxf(v, dpp_f<kDppRor8>(v));
    return fmaxf(fmaxf(rl_f(v, 0), rl_f(v, 16)), fmaxf(rl_f(v, 32), rl_f(v, 48)));
}
__device__ __forceinline__ float sum_groups_f(float v) {
    v += dpp_f<kDppRor8>(v);
    return (rl_f(v, 0) + rl_f(v, 16)) + (rl_f(v, 32) + rl_f(v, 48));
}

// ------------------------------------------------ wave-wide (DPP) ops ----
// Inclusive prefix sum over the 64 lanes: Hillis-Steele inside each row of
// 16 lanes (row_shr 1, 2, 4, 8), then row_bcast:15 and row_bcast:31 carry
// the row totals forward.
__device__ __forceinline__ unsigned wave_incl_scan(unsigned v) {
    int x = int(v);
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);
    return unsigned(x);
}
__device__ __forceinline__ unsigned wave_sum_u(unsigned v) {
    return unsigned(__builtin_amdgcn_readlane(int(wave_incl_scan(v)), 63));
}
// Butterfly inside rows of 16 lanes, then the four row results.
template <class Op>
__device__ __forceinline__ unsigned wave_reduce_u(unsigned v, Op op) {
    v = op(v, unsigned(dpp_i<kDppXor1>(int(v))));
    v = op(v, unsigned(dpp_i<kDppXor2>(int(v))));
    v = op(v, unsigned(dpp_i<kDppHalfMirror>(int(v))));
    v = op(v, unsigned(dpp_i<0x140>(int(v))));          // row_mirror
    const unsigned r0 = unsigned(__builtin_amdgcn_readlane(int(v), 0));
    const unsigned r1 = unsigned(__builtin_amdgcn_readlane(int(v), 16));
    const unsigned r2 = unsigned(__builtin_amdgcn_readlane(int(v), 32));
    const unsigned r3 = unsigned(__builtin_amdgcn_readlane(int(v), 48));
    return op(op(r0, r1), op(r2, r3));
}
__device__ __forceinline__ unsigned wave_max_u(unsigned v) {
    return wave_reduce_u(v, [](unsigned a, unsigned b) { return a > b ? a : b; });
}
__device__ __forceinline__ unsigned wave_min_u(unsigned v) {
    return wave_reduce_u(v, [](unsigned a, unsigned b) { return a < b ? a : b; });
}

__device__ __forceinline__ float wave_max_f(float v) {
    return __uint_as_float(wave_reduce_u(__float_as_uint(v), [](unsigned a, unsigned b) {
        return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
    }));
}
__device__ __forceinline__ float wave_sum_f(float v) {
    return __uint_as_float(wave_reduce_u(__float_as_uint(v), [](unsigned a, unsigned b) {
        return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
    }));
}

// Exclusive prefix sum over the block (NT threads, NT % 64 == 0, NT <= 1024).
// `tmp` holds NT/64 words of LDS; returns the block total in *total.
template <int NT>
__device__ __forceinline__ unsigned block_excl_scan(unsigned v, unsigned* tmp, unsigned* total) {
    constexpr int NW = NT / 64;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const unsigned incl = wave_incl_scan(v);
    if (lane == 63) tmp[wid] = incl;
    __syncthreads();
    unsigned before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const unsigned t = tmp[w];
        before += w < wid ? t : 0u;
        all += t;
    }
    *total = all;
    __syncthreads();
    return before + incl - v;
}

// ------------------------------------------------------- pipelines ----
// The work of one (request, KV head) -- a "pipeline" -- runs on one XCD.
// The dispatcher hands workgroups to the eight XCDs round robin, so the
// workgroups whose linear index agrees modulo 8 share an XCD and its L2:
// workgroup g serves pipeline (g % 8) + 8 m with m = (g / 8) / W, as its
// workgroup w = (g / 8) % W, where W is the launch's workgroups per
// pipeline.  Their hand-offs (the last-arriver tails below) meet in that
// L2, with no write-back of the cache to memory.  Every workgroup also
// records its XCD, so the last one can check that the pipeline stayed on
// one XCD (kFlagPlacement in the error flag otherwise).
constexpr int kXcds = 8;
constexpr int kTickInts = 128;        // per pipeline: one 8-byte ticket word, pipelines 512 bytes apart
constexpr int kMaxHandoffWgs = 4096;  // workgroups of one pipeline that the ticket word can count
constexpr int32_t kFlagBadLength = 1;
constexpr int32_t kFlagPlacement = 2;

// Workgroups of a launch with W workgroups per pipeline for BH pipelines.
__host__ __device__ constexpr int64_t pipe_grid(int W, int BH) {
    return int64_t(kXcds) * ((BH + kXcds - 1) / kXcds) * W;
}

struct PipeSlot {
    int bj;     // pipeline (request * Hkv + KV head), or -1: no work for this workgroup
    int w;      // workgroup index inside the pipeline
};
__device__ __forceinline__ PipeSlot pipe_slot(int W, int BH) {
    const int g = int(blockIdx.x);
    const int x = g % kXcds, k = g / kXcds;
    const int m = k / W, w = k - m * W;
    const int bj = x + kXcds * m;
    return PipeSlot{bj < BH ? bj : -1, w};
}

__device__ __forceinline__ int xcc_id() {
    int x;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(x));
    return x & 0xf;
}

// A request's length, read with a vector load: a plain load of this
// uniform address compiles to a scalar load, and the wait for it, shared
// with the kernel-argument loads, then sits in front of every load issued
// after it, adding one dependent memory round trip to the head of the
// kernel.  Here the wait falls where the length is first used.
__device__ __forceinline__ int32_t load_length(const int32_t* lengths, int b) {
    return __hip_atomic_load(lengths + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// The length from load_length, checked against [1, lmax] (0 when outside)
// at the point of this call: the compiler would otherwise move the first
// use of a uniform load, and the wait for it, up to the load itself; adding
// an opaque per-lane zero ties the use to this point.
__device__ __forceinline__ int64_t length_here(int32_t raw, int64_t lmax) {
    int32_t z;
    asm volatile("v_mov_b32 %0, 0" : "=v"(z));
    const int64_t x = int64_t(raw + z);
    return (x < 1 || x > lmax) ? 0 : x;
}

// Waits until this wave's vector stores (and atomics) have been acknowledged
// by the L2.
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Invalidates this compute unit's vector L1: a line it cached earlier in the
// launch (a neighbour of data it read) may be stale where another
// workgroup wrote since; after this, plain loads fetch from the XCD's L2.
__device__ __forceinline__ void inv_l1() { asm volatile("buffer_inv sc0" ::: "memory"); }

// Last-arriver hand-off of one pipeline's workgroups: each waits for its
// own stores, then takes a ticket; the workgroup with the last ticket gets
// true (in every thread) and continues with the pipeline's tail, after
// invalidating its L1 (so plain loads see what the others stored) and
// resetting the ticket word for the next launch.  No workgroup waits for
// another.  `word`: one int of LDS.
//
// The hand-off relies on one L2 for the whole pipeline, so the ticket also
// records where the workgroups ran: each adds 1 + (x << 16) + (x^2 << 32)
// to one 64-bit word, x its XCD.  With n tickets, count n, S1 = sum x and
// S2 = sum x^2, all x are equal exactly when n S2 = S1^2 (the variance is
// zero); otherwise the last workgroup sets kFlagPlacement.  Fields: count
// 16 bits, S1 16 bits (n <= kMaxHandoffWgs, x < 16), S2 32 bits.
__device__ __forceinline__ bool handoff_last(int32_t* tick, int nwg, int* word, int32_t* flag) {
    wait_stores();
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint64_t x = uint64_t(xcc_id());
        const uint64_t mine = 1ull | (x << 16) | ((x * x) << 32);
        uint64_t* t = reinterpret_cast<uint64_t*>(tick);
        const uint64_t all = __hip_atomic_fetch_add(t, mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + mine;
        const bool last = int(all & 0xffffu) == nwg;
        *word = last;
        if (last) {
            __hip_atomic_store(t, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const uint64_t s1 = (all >> 16) & 0xffffu, s2 = all >> 32;
            if (uint64_t(nwg) * s2 != s1 * s1) atomicOr(flag, kFlagPlacement);
        }
    }
    __syncthreads();
    const bool last = *word != 0;
    if (last) inv_l1();
    return last;
}

// |x| of the two bf16 values of a dword, as bit patterns; max of the two.
__device__ __forceinline__ unsigned abs_bits2(uint32_t w) {
    return max(w & 0x7fffu, (w >> 16) & 0x7fffu);
}

// ---------------------------------------------------------------------------
// Query: one absmax scale per query head, codes with the same rounding as the
// keys, and the group sum Q_j over the G query heads of KV head j (GQA
// table of "KV Cache 与长上下文推理", section "KV Cache 压缩技术").
// Wave w < G handles query head j*G + w; lane l handles dims 2l and 2l+1.
// Qlds must hold 128 ints; the caller's block has at least G waves.
// ---------------------------------------------------------------------------
// This thread's bf16 pair of the query (wave w < G: head j*G + w, dims 2l
// and 2l + 1), loaded early so that the codes can be formed while other
// loads are in flight.
__device__ __forceinline__ uint32_t query_pair(const uint16_t* __restrict__ q_b, int j, int G) {
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    return w < G ? reinterpret_cast<const uint32_t*>(q_b + (j * G + w) * kHeadDim)[lane] : 0u;
}

__device__ __forceinline__ void group_query_codes(uint32_t pr, int j, int G, int* Qlds, int8_t* __restrict__ q8_b) {
    if (threadIdx.x < kHeadDim) Qlds[threadIdx.x] = 0;
    __syncthreads();
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (w < G) {
        const int h = j * G + w;
        const unsigned ab = wave_max_u(abs_bits2(pr));
        const float amax = bf16_to_f32(uint16_t(ab));
        const int c0 = code_of(bf16_lo(pr), amax), c1 = code_of(bf16_hi(pr), amax);
        atomicAdd(Qlds + 2 * lane, c0);
        atomicAdd(Qlds + 2 * lane + 1, c1);
        if (q8_b) {
            uint16_t two = uint16_t((uint32_t(c0) & 0xffu) | ((uint32_t(c1) & 0xffu) << 8));
            reinterpret_cast<uint16_t*>(q8_b + h * kHeadDim)[lane] = two;
        }
    }
    __syncthreads();
}
__device__ __forceinline__ void group_query_codes(const uint16_t* __restrict__ q_b, int j, int G, int* Qlds,
                                                  int8_t* __restrict__ q8_b) {
    group_query_codes(query_pair(q_b, j, G), j, G, Qlds, q8_b);
}

}  // namespace sd
