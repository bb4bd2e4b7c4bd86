// Library-internal context and kernel launchers.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

#include "sd.h"

namespace sd {

// Per-stage launch geometry.
struct StageGeom {
    int chunk, stride, keep;
    int nsamp;          // samples per chunk = chunk / stride
    int ncand;          // candidates per (request, KV head)
    int koff;           // offset of this stage in kept_idx
    int per_wg;         // candidates scored per workgroup
    int nwg;            // workgroups per (request, KV head)
    int nrows;          // key rows read per candidate (nsamp, or more when the next stage is fused in)
    int rstride;        // their token stride
};

// Geometry of one stage as the kernels see it.
struct StageDev {
    int chunk, stride, keep, nsamp, ncand, koff;
    int ratio;      // children per parent chunk (chunk of stage s-1 / chunk of stage s); 1 for stage 0
};

constexpr int kVcCounters = 16;
// Decode splits per (request, KV head): at most 64 (one per lane of the
// merge's weight pass).  With many (request, KV head) pipelines the decode
// runs "wide": at most kDecodeWideSplits splits, about kDecodeWideWgs
// workgroups in all, and a kernel whose merge sizes its loads for that many
// splits (fewer registers, three workgroups per CU instead of two).
constexpr int kDecodeMaxSplits = 64;
constexpr int kDecodeWideSplits = 48;
constexpr int kDecodeWideWgs = 768;
constexpr int kDecodeWideMinPipes = 32;
// Candidates per wave of a pruning kernel, at most: one batch of 8 row
// loads, or two for the stages after the first with many pipelines.
constexpr int kMaxCandPerWave = 16;
// Value caches of at most kVcOnchipSlots slots and kVcOnchipBlocks attended
// blocks per (request, KV head) take the LRU step with its working state on
// chip (sd_vcache.hip).
constexpr int kVcOnchipSlots = 8192;
constexpr int kVcOnchipBlocks = 1024;
// Entry of the per-step block -> slot map: the slot in the low 24 bits, a
// miss (block not resident: read it from host memory into its slot) or a
// refill (resident, but written when fewer of its rows were below the
// length than now: read it again) in the flag bits.
constexpr int32_t kVcMissBit = int32_t(0x40000000);
constexpr int32_t kVcRefillBit = int32_t(0x20000000);
constexpr int32_t kVcSlotMask = int32_t(0x00ffffff);

// Device-side state of the host-value path (values_on_host = 1).
struct ValueCache {
    int32_t slots;          // slots (8-token blocks) per (request, KV head)
    int32_t nblk_max;       // ceil(Lmax / 8): page-table entries per (b, j)
    uint16_t* pool;         // [B][Hkv][slots][8][d] bf16 value blocks
    int32_t* page;          // [B][Hkv][nblk_max] slot of a block or -1
    int32_t* slot_block;    // [B][Hkv][slots] block held by a slot or -1
    int32_t* slot_last;     // [B][Hkv][slots] last step the slot was used
    int32_t* used;          // [B][Hkv] slots filled so far
    int32_t* order;         // [2][B][Hkv][slots] recency order (oldest first), double buffered
    int32_t* evicted;       // [B][Hkv][max_blocks] slots evicted this step, oldest first
    int32_t* blk_slot;      // [B][Hkv][max_blocks] slot of each attended block (| kVcMissBit, | kVcRefillBit)
    int32_t* slot_fill;     // [B][Hkv][slots] rows of its block a slot holds (those below the length when filled)
    int32_t* stepc;         // [B][Hkv] steps applied since the reset (the LRU's clock, kept on the device)
    int64_t* counters;      // [16]: steps, needed, hits, misses, then per step parity p:
                            //       [4+4p] needed, [5+4p] hits, [6+4p] misses, [7+4p] refills;
                            //       [12] refills over all steps
};

}  // namespace sd

struct sd_ctx {
    sd_config cfg;
    int device;
    int G;                  // query heads per KV head
    int S;                  // stages
    int64_t Lmax;
    int keep_total;
    int max_blocks;         // attended 8-token blocks per (request, KV head)
    int nsplit;             // flash-decode splits per (request, KV head)
    int nsplit_a;           // of which cover the sink/window blocks (device values only)
    int decode_wide;        // many pipelines: at most kDecodeWideSplits splits, the wide decode kernel
    int nsplit_d;           // splits per (request, KV head) of the dense decode (sd_dense_decode)
    int64_t sketch_rows;    // rows per (request, KV head) of the int4 first-stage sketch: ceil(Lmax / r_1)
    float scale_log2;       // softmax_scale * log2(e)
    sd::StageGeom st[SD_MAX_STAGES];
    size_t select_lds;      // dynamic LDS bytes of the stage kernels

    // device workspace (one allocation)
    void* ws;
    size_t ws_bytes;
    int32_t* scores[SD_MAX_STAGES];   // [B][Hkv][ncand]
    int32_t* qgroup;                  // [B][Hkv][d] group query sums
    uint32_t* blocks;                 // [B][Hkv][max_blocks] (block << 8) | token mask
    int32_t* nblocks;                 // [B][Hkv]
    float* part;                      // acc [B*Hkv][n][G][d], then (m, l) [B*Hkv][n][G][2], n = the
                                      // launch's splits (nsplit, or nsplit_d for the dense decode)
    // fused last stage: the kernel of stage S-2 also scores every child chunk
    // of every stage S-2 candidate for stage S-1 (reading all rows stage S-1
    // samples), and the decode kernel selects stage S-2, gathers the kept
    // children's scores and selects stage S-1; no kernel runs for stage S-1
    int fuse;
    int fuse_rq;                      // children per stage S-2 chunk
    int fuse_m;                       // stage S-2 stride / stage S-1 stride
    int32_t* pre;                     // [B][Hkv][st[S-2].ncand * fuse_rq] children's stage S-1 scores
                                      // (half: [st[S-2].ncand * half_rq] maxima over the rows stage S-2 read)
    int half;                         // unfused, stage S-2's stride twice stage S-1's (8 rows per chunk):
                                      // stage S-1 reads only the rows stage S-2 did not
    int half_rq;                      // children per stage S-2 chunk (half)
    unsigned* absmax_bits;            // [B][Hkv] bf16 bits of each key scale (sd_quantize_keys, sd_append_kv)
    int32_t* requant;                 // [B][Hkv] set by sd_append_kv when the scale grew
    int32_t* tick;                    // [B*Hkv][kTickInts] last-arriver counters (zero between launches)
    int32_t* flag;                    // device error flag (kFlagBadLength | kFlagPlacement), right after tick
    uint32_t* rec;                    // caller's attended-word record (sd_record_attended), or null
    // gathered-copy value fetch (SD_VALUE_FETCH_COPY)
    int vfetch;                       // SD_VALUE_FETCH_*
    hipStream_t vside;                // side stream of the copies (default priority)
    hipEvent_t vside_done;            // recorded after a step's copies
    int32_t* vstage;                  // pinned host staging: nblocks [BH], lengths [B], blocks and blk_slot [BH][max_blocks]
    int64_t vcopies;                  // copies (runs) enqueued by the last step
    sd::ValueCache vc;
    int vc_onchip;                    // the LRU step keeps its working state on chip (small caches)
    const void* vhost_key;            // last host value pointer seen, and its device alias
    const uint16_t* vhost_dev;
    // profiling (sd_profile_start / sd_profile_stop)
    uint32_t prof_mask;
    int32_t prof_max, prof_n;
    hipEvent_t* prof_ev;              // [2 * prof_max]
    int8_t* prof_kind;                // [prof_max]
};

namespace sd {

// Optional profiling timestamps carried by a kernel dispatch itself
// (hipExtLaunchKernelGGL), so that timing adds no marker packets between
// kernels.  start/stop may each be null.
struct Timing {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
};

template <typename... KArgs, typename... Args>
inline void launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t lds, hipStream_t s, Timing t,
                   Args&&... args) {
    if (t.start || t.stop)
        hipExtLaunchKernelGGL(kernel, grid, block, uint32_t(lds), s, t.start, t.stop, 0u, std::forward<Args>(args)...);
    else
        kernel<<<grid, block, lds, s>>>(std::forward<Args>(args)...);
}

hipError_t launch_quantize_keys(sd_ctx* c, const uint16_t* k, const int32_t* lengths, int8_t* k8,
                                float* absmax, hipStream_t s, Timing t = {});
// Appends n rows per (request, KV head) at lengths[b] and recodes the rows of
// the (request, KV head)s whose key scale grew.
hipError_t launch_append(sd_ctx* c, const uint16_t* k_new, const uint16_t* v_new, int n, const int32_t* lengths,
                         uint16_t* k, int8_t* k8, uint16_t* v, uint8_t* k4, float* absmax, hipStream_t s,
                         Timing t = {});
hipError_t launch_quantize_query(sd_ctx* c, const uint16_t* q, int8_t* q8, int32_t* qg, hipStream_t s);
// given: the kept set that the launch would select (stage - 1's for a
// pruning stage, the last stage's for the decode and value-cache kernels)
// is read from kept_idx instead, where an earlier step left it.
// fused: this step runs the fused plan (the stage before the last also
// scores the last stage's candidates, and the decode kernel selects both).
// k4: the int4 sketch of the first stage's rows (stage 0 scores it in place
// of k8), or null.
hipError_t launch_prune_stage(sd_ctx* c, int stage, bool given, bool fused, const uint16_t* q, const int8_t* k8,
                              const uint8_t* k4, const int32_t* lengths, int32_t* kept, hipStream_t s,
                              Timing t = {});
// int4 sketch rows of the first stage (codes with the stored key scales).
hipError_t launch_sketch4(sd_ctx* c, const uint16_t* k, const int32_t* lengths, uint8_t* k4, hipStream_t s);
// Attention over the attended set (the last stage's kept set, sink and
// window), the splits merged into `out` by the last split of each (request,
// KV head) to finish.
hipError_t launch_attend(sd_ctx* c, bool given, bool fused, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                         const int32_t* lengths, int32_t* kept, uint16_t* out, hipStream_t s, Timing t = {});
// Merges `nsplit` split partials per (request, KV head) into the bf16 output
// (the dense decode's merge).
hipError_t launch_combine(sd_ctx* c, int nsplit, uint16_t* out, hipStream_t s, Timing t = {});
// Dense decode over every token t < L_b (split partials; launch_combine
// with c->nsplit_d merges them).
hipError_t launch_dense(sd_ctx* c, const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* lengths,
                        hipStream_t s, Timing t = {});
hipError_t launch_value_cache_update(sd_ctx* c, bool given, bool fused, const int32_t* lengths, int32_t* kept,
                                     hipStream_t s, Timing t = {});
hipError_t launch_value_cache_reset(sd_ctx* c, hipStream_t s);
StageDev stage_dev(const sd_ctx* c, int st);

}  // namespace sd
