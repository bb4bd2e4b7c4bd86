// Symmetric int8 quantisation of the key cache and of the step's query.
//
// Keys: one absmax scale per (request, KV head) over its valid rows; codes
// rint(127 k / a).  Sources: summary page of "HCAttention: Extreme KV cache
// compression via heterogeneous attention computing for LLMs", section 引言
// (keys quantised and kept on the GPU for scoring); page "KV Cache 与长上下文
// 推理", section "KV Cache 压缩技术" (INT8 key cache).
//
// Both passes stream the bf16 cache with 16-byte loads, 16 lanes per
// 256-byte row.  The absmax pass works on bf16 bit patterns (|x| ordering is
// the ordering of the low 15 bits for finite values).
#include <algorithm>

#include "sd_device.h"
#include "sd_internal.h"

namespace sd {

namespace {

constexpr int kQuantThreads = 256;
constexpr int kQuantRowsPerWg = 1024;     // 256 KiB of bf16 keys per workgroup

__global__ void sd_absmax_init_kernel(unsigned* absmax_bits, int n) {
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) absmax_bits[i] = 0u;
}

__global__ __launch_bounds__(kQuantThreads) void sd_absmax_kernel(
    const uint16_t* __restrict__ k, const int32_t* __restrict__ lengths, int64_t Lmax, int Hkv,
    unsigned* __restrict__ absmax_bits, int32_t* __restrict__ flag) {
    const int bj = blockIdx.y, b = bj / Hkv;
    const int64_t L = lengths[b];
    if (L < 1 || L > Lmax) {
        if (blockIdx.x == 0 && threadIdx.x == 0) atomicOr(flag, 1);
        return;
    }
    const int64_t r0 = int64_t(blockIdx.x) * kQuantRowsPerWg;
    const int64_t r1 = min(r0 + kQuantRowsPerWg, L);
    if (r0 >= r1) return;
    const u32x4* base = reinterpret_cast<const u32x4*>(k + int64_t(bj) * Lmax * kHeadDim);
    const int64_t e0 = r0 * 16, e1 = r1 * 16;   // 16 u32x4 per row
    unsigned m = 0;
    int64_t e = e0 + threadIdx.x;
    for (; e + 3 * kQuantThreads < e1; e += 4 * kQuantThreads) {
        u32x4 w0 = __builtin_nontemporal_load(base + e);
        u32x4 w1 = __builtin_nontemporal_load(base + e + kQuantThreads);
        u32x4 w2 = __builtin_nontemporal_load(base + e + 2 * kQuantThreads);
        u32x4 w3 = __builtin_nontemporal_load(base + e + 3 * kQuantThreads);
        m = max(m, max(max(abs_bits2(w0.x), abs_bits2(w0.y)), max(abs_bits2(w0.z), abs_bits2(w0.w))));
        m = max(m, max(max(abs_bits2(w1.x), abs_bits2(w1.y)), max(abs_bits2(w1.z), abs_bits2(w1.w))));
        m = max(m, max(max(abs_bits2(w2.x), abs_bits2(w2.y)), max(abs_bits2(w2.z), abs_bits2(w2.w))));
        m = max(m, max(max(abs_bits2(w3.x), abs_bits2(w3.y)), max(abs_bits2(w3.z), abs_bits2(w3.w))));
    }
    for (; e < e1; e += kQuantThreads) {
        u32x4 w = base[e];
        m = max(m, max(max(abs_bits2(w.x), abs_bits2(w.y)), max(abs_bits2(w.z), abs_bits2(w.w))));
    }
    m = wave_max_u(m);
    __shared__ unsigned red[kQuantThreads / kWave];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned r = red[0];
        for (int i = 1; i < kQuantThreads / kWave; ++i) r = max(r, red[i]);
        atomicMax(absmax_bits + bj, r);
    }
}

__device__ __forceinline__ uint32_t pack4(int a, int b, int c, int d) {
    return (uint32_t(a) & 0xffu) | ((uint32_t(b) & 0xffu) << 8) | ((uint32_t(c) & 0xffu) << 16) |
           (uint32_t(d) << 24);
}

__device__ __forceinline__ uint2 codes8(u32x4 w, float a) {
    uint2 r;
    r.x = pack4(code_of(bf16_lo(w.x), a), code_of(bf16_hi(w.x), a), code_of(bf16_lo(w.y), a),
                code_of(bf16_hi(w.y), a));
    r.y = pack4(code_of(bf16_lo(w.z), a), code_of(bf16_hi(w.z), a), code_of(bf16_lo(w.w), a),
                code_of(bf16_hi(w.w), a));
    return r;
}

// Codes of rows [0, lengths[b] + len_add) with the stored scale; workgroup
// x takes row tiles x, x + gridDim.x, ...  With `only` set, a (request, KV
// head) whose only[bj] is 0 is skipped (the append's requantisation).
__global__ __launch_bounds__(kQuantThreads) void sd_quantize_kernel(
    const uint16_t* __restrict__ k, const int32_t* __restrict__ lengths, int len_add, int64_t Lmax, int Hkv,
    const unsigned* __restrict__ absmax_bits, const int32_t* __restrict__ only, int8_t* __restrict__ k8,
    float* __restrict__ absmax_out) {
    const int bj = blockIdx.y, b = bj / Hkv;
    if (only && only[bj] == 0) return;
    const int64_t L = int64_t(lengths[b]) + len_add;
    if (L < 1 || L > Lmax) return;
    const float a = bf16_to_f32(uint16_t(absmax_bits[bj]));
    if (absmax_out && blockIdx.x == 0 && threadIdx.x == 0) absmax_out[bj] = a;
    const u32x4* src = reinterpret_cast<const u32x4*>(k + int64_t(bj) * Lmax * kHeadDim);
    uint2* dst = reinterpret_cast<uint2*>(k8 + int64_t(bj) * Lmax * kHeadDim);
    for (int64_t r0 = int64_t(blockIdx.x) * kQuantRowsPerWg; r0 < L; r0 += int64_t(gridDim.x) * kQuantRowsPerWg) {
        const int64_t r1 = min(r0 + kQuantRowsPerWg, L);
        const int64_t e0 = r0 * 16, e1 = r1 * 16;
        int64_t e = e0 + threadIdx.x;
        for (; e + kQuantThreads < e1; e += 2 * kQuantThreads) {
            u32x4 w0 = __builtin_nontemporal_load(src + e);
            u32x4 w1 = __builtin_nontemporal_load(src + e + kQuantThreads);
            dst[e] = codes8(w0, a);
            dst[e + kQuantThreads] = codes8(w1, a);
        }
        for (; e < e1; e += kQuantThreads) dst[e] = codes8(src[e], a);
    }
}

// int4 sketch of the first pruning stage's rows: for t = i * stride < L,
// row i of the sketch holds the 4-bit codes of key row t with the stored
// scale, as two's-complement nibbles, channel 2m in the low and channel
// 2m + 1 in the high nibble of byte m (64 bytes per row).  16 threads per
// row, each codes 8 channels (one 16-byte load) into one 4-byte word.
__device__ __forceinline__ uint32_t sketch_word(u32x4 w, float a) {
    const uint32_t x[4] = {w.x, w.y, w.z, w.w};
    uint32_t word = 0;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const uint32_t lo = uint32_t(code4_of(bf16_lo(x[m]), a)) & 0xfu;
        const uint32_t hi = uint32_t(code4_of(bf16_hi(x[m]), a)) & 0xfu;
        word |= (lo | (hi << 4)) << (8 * m);
    }
    return word;
}

// Rows of t < lengths[b] + len_add; with `only` set, a (request, KV head)
// whose only[bj] is 0 is skipped (the append's recoding).
__global__ __launch_bounds__(kQuantThreads) void sd_sketch4_kernel(
    const uint16_t* __restrict__ k, const int32_t* __restrict__ lengths, int len_add, int64_t Lmax, int Hkv,
    int stride, int64_t rows, const unsigned* __restrict__ absmax_bits, const int32_t* __restrict__ only,
    uint8_t* __restrict__ k4) {
    const int bj = blockIdx.y, b = bj / Hkv;
    if (only && only[bj] == 0) return;
    const int64_t L = int64_t(lengths[b]) + len_add;
    if (L < 1 || L > Lmax) return;
    const float a = bf16_to_f32(uint16_t(absmax_bits[bj]));
    const int64_t n = (L + stride - 1) / stride;             // sketch rows of this request
    const u32x4* src = reinterpret_cast<const u32x4*>(k + int64_t(bj) * Lmax * kHeadDim);
    uint32_t* dst = reinterpret_cast<uint32_t*>(k4 + int64_t(bj) * rows * (kHeadDim / 2));
    const int sub = threadIdx.x & 15;
    for (int64_t i = int64_t(blockIdx.x) * kQuantRowsPerWg + (threadIdx.x >> 4);
         i < min(n, int64_t(blockIdx.x + 1) * kQuantRowsPerWg); i += kQuantThreads / 16) {
        dst[i * 16 + sub] = sketch_word(src[i * stride * 16 + sub], a);
    }
}

// Appends n rows per (request, KV head) at t = L_b .. L_b + n - 1: copies
// the new bf16 keys and values into the caches and codes the new keys with
// a' = max(a, absmax of the new keys), a being the scale stored for the
// cache.  Stores a' and sets requant[bj] when a' > a (the earlier rows are
// then recoded by sd_quantize_kernel with `only` = requant).  One workgroup
// per (request, KV head), so the scale is read and written by one
// workgroup.  A request with L_b < 1 or L_b + n > Lmax is left untouched and
// raises the flag.
__global__ __launch_bounds__(kQuantThreads) void sd_append_kernel(
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new, int n,
    const int32_t* __restrict__ lengths, int64_t Lmax, int Hkv, uint16_t* __restrict__ k, int8_t* __restrict__ k8,
    uint16_t* __restrict__ v, unsigned* __restrict__ absmax_bits, int32_t* __restrict__ requant,
    float* __restrict__ absmax_out, int32_t* __restrict__ flag, uint8_t* __restrict__ k4, int stride4,
    int64_t rows4) {
    const int j = blockIdx.x, b = blockIdx.y, bj = b * Hkv + j;
    const int64_t L = lengths[b];
    if (L < 1 || L > Lmax - n) {
        if (threadIdx.x == 0) {
            requant[bj] = 0;
            if (j == 0) atomicOr(flag, 1);
        }
        return;
    }
    const u32x4* ks = reinterpret_cast<const u32x4*>(k_new + int64_t(bj) * n * kHeadDim);
    const u32x4* vs = reinterpret_cast<const u32x4*>(v_new + int64_t(bj) * n * kHeadDim);
    const int64_t ne = int64_t(n) * 16;        // 16 u32x4 per row
    unsigned m = 0;
    for (int64_t e = threadIdx.x; e < ne; e += kQuantThreads) {
        const u32x4 w = ks[e];
        m = max(m, max(max(abs_bits2(w.x), abs_bits2(w.y)), max(abs_bits2(w.z), abs_bits2(w.w))));
    }
    m = wave_max_u(m);
    __shared__ unsigned red[kQuantThreads / kWave];
    __shared__ unsigned anew;
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned r = absmax_bits[bj];
        const unsigned old = r;
        for (int i = 0; i < kQuantThreads / kWave; ++i) r = max(r, red[i]);
        absmax_bits[bj] = r;
        requant[bj] = r > old ? 1 : 0;
        if (absmax_out) absmax_out[bj] = bf16_to_f32(uint16_t(r));
        anew = r;
    }
    __syncthreads();
    const float a = bf16_to_f32(uint16_t(anew));
    u32x4* kd = reinterpret_cast<u32x4*>(k + (int64_t(bj) * Lmax + L) * kHeadDim);
    u32x4* vd = reinterpret_cast<u32x4*>(v + (int64_t(bj) * Lmax + L) * kHeadDim);
    uint2* k8d = reinterpret_cast<uint2*>(k8 + (int64_t(bj) * Lmax + L) * kHeadDim);
    uint32_t* k4d = k4 ? reinterpret_cast<uint32_t*>(k4 + int64_t(bj) * rows4 * (kHeadDim / 2)) : nullptr;
    for (int64_t e = threadIdx.x; e < ne; e += kQuantThreads) {
        const u32x4 w = ks[e];
        kd[e] = w;
        k8d[e] = codes8(w, a);
        vd[e] = vs[e];
        const int64_t t = L + e / 16;             // token of this word
        if (k4d && t % stride4 == 0) k4d[(t / stride4) * 16 + e % 16] = sketch_word(w, a);
    }
}

}  // namespace

namespace {

__global__ __launch_bounds__(256) void sd_quantize_query_kernel(const uint16_t* __restrict__ q, int Hq,
                                                                int Hkv, int G, int8_t* __restrict__ q8,
                                                                int32_t* __restrict__ qg) {
    __shared__ int Qlds[kHeadDim];
    const int j = blockIdx.x, b = blockIdx.y;
    group_query_codes(q + int64_t(b) * Hq * kHeadDim, j, G, Qlds, q8 ? q8 + int64_t(b) * Hq * kHeadDim : nullptr);
    if (qg && threadIdx.x < kHeadDim) qg[(int64_t(b) * Hkv + j) * kHeadDim + threadIdx.x] = Qlds[threadIdx.x];
}

}  // namespace

hipError_t launch_quantize_keys(sd_ctx* c, const uint16_t* k, const int32_t* lengths, int8_t* k8,
                                float* absmax, hipStream_t s, Timing t) {
    const int BH = c->cfg.batch * c->cfg.num_kv_heads;
    launch(sd_absmax_init_kernel, dim3((BH + 255) / 256), dim3(256), 0, s, Timing{t.start, nullptr},
           c->absmax_bits, BH);
    const int nwg = int((c->Lmax + kQuantRowsPerWg - 1) / kQuantRowsPerWg);
    dim3 grid(nwg, BH);
    launch(sd_absmax_kernel, grid, dim3(kQuantThreads), 0, s, Timing{}, k, lengths, c->Lmax,
           c->cfg.num_kv_heads, c->absmax_bits, c->flag);
    launch(sd_quantize_kernel, grid, dim3(kQuantThreads), 0, s, Timing{nullptr, t.stop}, k, lengths, 0, c->Lmax,
           c->cfg.num_kv_heads, (const unsigned*)c->absmax_bits, (const int32_t*)nullptr, k8, absmax);
    return hipGetLastError();
}

hipError_t launch_sketch4(sd_ctx* c, const uint16_t* k, const int32_t* lengths, uint8_t* k4, hipStream_t s) {
    const int BH = c->cfg.batch * c->cfg.num_kv_heads;
    const int64_t rows = c->sketch_rows;
    const int nwg = int((rows + kQuantRowsPerWg - 1) / kQuantRowsPerWg);
    launch(sd_sketch4_kernel, dim3(nwg, BH), dim3(kQuantThreads), 0, s, Timing{}, k, lengths, 0, c->Lmax,
           c->cfg.num_kv_heads, c->st[0].stride, rows, (const unsigned*)c->absmax_bits, (const int32_t*)nullptr, k4);
    return hipGetLastError();
}

hipError_t launch_append(sd_ctx* c, const uint16_t* k_new, const uint16_t* v_new, int n, const int32_t* lengths,
                         uint16_t* k, int8_t* k8, uint16_t* v, uint8_t* k4, float* absmax, hipStream_t s, Timing t) {
    const int BH = c->cfg.batch * c->cfg.num_kv_heads;
    launch(sd_append_kernel, dim3(c->cfg.num_kv_heads, c->cfg.batch), dim3(kQuantThreads), 0, s,
           Timing{t.start, nullptr}, k_new, v_new, n, lengths, c->Lmax, c->cfg.num_kv_heads, k, k8, v,
           c->absmax_bits, c->requant, absmax, c->flag, k4, c->st[0].stride, c->sketch_rows);
    // recoding of every row of the (request, KV head)s whose scale grew: at
    // most 64 workgroups per (request, KV head), each looping over row tiles
    // (the others exit at once); then their sketch rows
    const int ntile = int((c->Lmax + kQuantRowsPerWg - 1) / kQuantRowsPerWg);
    launch(sd_quantize_kernel, dim3(std::min(ntile, 64), BH), dim3(kQuantThreads), 0, s,
           Timing{nullptr, k4 ? nullptr : t.stop}, (const uint16_t*)k, lengths, n, c->Lmax, c->cfg.num_kv_heads,
           (const unsigned*)c->absmax_bits, (const int32_t*)c->requant, k8, (float*)nullptr);
    if (k4) {
        const int nwg4 = int((c->sketch_rows + kQuantRowsPerWg - 1) / kQuantRowsPerWg);
        launch(sd_sketch4_kernel, dim3(nwg4, BH), dim3(kQuantThreads), 0, s, Timing{nullptr, t.stop},
               (const uint16_t*)k, lengths, n, c->Lmax, c->cfg.num_kv_heads, c->st[0].stride, c->sketch_rows,
               (const unsigned*)c->absmax_bits, (const int32_t*)c->requant, k4);
    }
    return hipGetLastError();
}

hipError_t launch_quantize_query(sd_ctx* c, const uint16_t* q, int8_t* q8, int32_t* qg, hipStream_t s) {
    dim3 grid(c->cfg.num_kv_heads, c->cfg.batch);
    sd_quantize_query_kernel<<<grid, 256, 0, s>>>(q, c->cfg.num_q_heads, c->cfg.num_kv_heads, c->G, q8, qg);
    return hipGetLastError();
}

}  // namespace sd
