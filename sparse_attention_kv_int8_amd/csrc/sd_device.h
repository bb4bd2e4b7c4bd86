// Device helpers shared by the sparse decode kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sd {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
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
__device__ __forceinline__ void group_query_codes(const uint16_t* __restrict__ q_b, int j, int G, int* Qlds,
                                  int8_t* __restrict__ q8_b) {
    if (threadIdx.x < kHeadDim) Qlds[threadIdx.x] = 0;
    __syncthreads();
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (w < G) {
        const int h = j * G + w;
        const uint32_t pr = reinterpret_cast<const uint32_t*>(q_b + h * kHeadDim)[lane];
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

}  // namespace sd
