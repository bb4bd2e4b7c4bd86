// Host side of the C ABI declared in include/sd.h: validation, launch
// geometry, the one workspace allocation, and the entry points.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>

#include "sd_device.h"
#include "sd_internal.h"
#include "sd_select.h"

// Workspace of sd_decode_step_noalloc, for callers that cannot allocate:
// a fixed array in device memory, one copy on every GPU the library runs on,
// held until the process ends.  Host code never passes its name to a
// kernel (in host code the name is a stand-in, not a device address): the
// device address of each GPU's copy is looked up once with
// hipGetSymbolAddress and used from then on.
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxCandidates = 15872;   // per-stage candidates (+ keep) held in LDS by the select
constexpr int kMaxSamples = 64;         // chunk / stride

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

thread_local char g_last_error[256];

sd_status from_hip(hipError_t e, const char* where = "HIP call") {
    if (e == hipSuccess) return SD_OK;
    std::snprintf(g_last_error, sizeof(g_last_error), "%s: %s (%d)", where, hipGetErrorString(e), int(e));
    if (e == hipErrorOutOfMemory) return SD_ERR_OUT_OF_MEMORY;
    return SD_ERR_HIP;
}

// Validates the configuration and fills the geometry of `c` (no HIP calls).
sd_status plan(const sd_config& cfg, sd_ctx* c) {
    if (cfg.batch < 1 || cfg.num_kv_heads < 1 || cfg.num_q_heads < 1) return SD_ERR_INVALID_ARG;
    if (cfg.num_q_heads % cfg.num_kv_heads != 0) return SD_ERR_INVALID_ARG;
    const int G = cfg.num_q_heads / cfg.num_kv_heads;
    if (G != 1 && G != 2 && G != 4) return SD_ERR_UNSUPPORTED;
    if (cfg.head_dim != sd::kHeadDim) return SD_ERR_UNSUPPORTED;
    if (cfg.max_context < 1 || cfg.max_context > (int64_t(1) << 31) - 8) return SD_ERR_INVALID_ARG;
    if (cfg.num_stages < 1 || cfg.num_stages > SD_MAX_STAGES) return SD_ERR_INVALID_ARG;
    if (cfg.sink < 0 || cfg.window < 0) return SD_ERR_INVALID_ARG;
    if (!(cfg.softmax_scale >= 0.0f) || !std::isfinite(cfg.softmax_scale)) return SD_ERR_INVALID_ARG;
    if (cfg.values_on_host != 0 && cfg.values_on_host != 1) return SD_ERR_INVALID_ARG;
    if (int64_t(cfg.batch) * cfg.num_kv_heads > 65535) return SD_ERR_UNSUPPORTED;

    c->cfg = cfg;
    c->G = G;
    c->S = cfg.num_stages;
    c->Lmax = cfg.max_context;
    int koff = 0;
    for (int s = 0; s < cfg.num_stages; ++s) {
        const sd_stage& in = cfg.stage[s];
        if (in.chunk < 1 || in.stride < 1 || in.keep < 1) return SD_ERR_INVALID_ARG;
        if (in.chunk % in.stride != 0) return SD_ERR_INVALID_ARG;
        if (s > 0 && cfg.stage[s - 1].chunk % in.chunk != 0) return SD_ERR_INVALID_ARG;
        sd::StageGeom& g = c->st[s];
        g.chunk = in.chunk;
        g.stride = in.stride;
        g.keep = in.keep;
        g.nsamp = in.chunk / in.stride;
        if (g.nsamp > kMaxSamples) return SD_ERR_UNSUPPORTED;
        const int64_t nc = s == 0 ? (cfg.max_context + in.chunk - 1) / in.chunk
                                  : int64_t(cfg.stage[s - 1].keep) * (cfg.stage[s - 1].chunk / in.chunk);
        if (nc + in.keep > kMaxCandidates) return SD_ERR_UNSUPPORTED;
        if (in.keep > kMaxCandidates) return SD_ERR_UNSUPPORTED;
        g.ncand = int(nc);
        g.koff = koff;
        koff += in.keep;
        // candidates per workgroup: 4 waves x (one or two batches of 8 row loads)
        const int ns8 = (g.nsamp + 7) / 8;
        const int ns8p = ns8 == 1 ? 1 : ns8 == 2 ? 2 : ns8 <= 4 ? 4 : 8;
        const int cb = ns8p >= 8 ? 1 : 8 / ns8p;
        const int cpw = cb;
        g.per_wg = 4 * cpw;
        g.nwg = (g.ncand + g.per_wg - 1) / g.per_wg;
        g.nrows = g.nsamp;
        g.rstride = g.stride;
    }
    if (cfg.stage[cfg.num_stages - 1].chunk % 8 != 0) return SD_ERR_UNSUPPORTED;
    if (koff > 65535) return SD_ERR_UNSUPPORTED;
    c->keep_total = koff;
    c->sketch_rows = (cfg.max_context + cfg.stage[0].stride - 1) / cfg.stage[0].stride;
    const sd_stage& last = cfg.stage[cfg.num_stages - 1];
    const int64_t mb = int64_t(last.keep) * (last.chunk / 8) + (cfg.sink + 7) / 8 + (cfg.window + 7) / 8 + 1;
    if (mb > (int64_t(1) << 20)) return SD_ERR_UNSUPPORTED;
    c->max_blocks = int(mb);
    const int BH = cfg.batch * cfg.num_kv_heads;
    // Decode splits per (request, KV head): about 512 workgroups in all, at
    // most 48 per (request, KV head) with device values (the merge reads
    // every split's partial: at B = 1, 48 splits measured about 1 us faster
    // per step than 64 at 128K and at 1M; 32 and 40 were no faster than
    // 64) and 64 with host values (whose decode waits on host reads: 48
    // measured 6 us slower per step on the 3M sequence), at most one per 4
    // attended blocks.
    // With at least kDecodeWideMinPipes pipelines (device values), about
    // kDecodeWideWgs workgroups and the wide kernel instead: its merge sizes
    // its loads for at most kDecodeWideSplits splits, which leaves room for
    // three workgroups per CU.  16 requests of up to 128K: 6 splits per
    // (request, KV head), the decode kernel 60 -> 48 us.  (At B = 1 the
    // wide kernel measured 1.2 us slower per step: the compiler schedules
    // its other code for the higher occupancy.)
    c->decode_wide = !cfg.values_on_host && BH >= sd::kDecodeWideMinPipes;
    int ns = ((c->decode_wide ? sd::kDecodeWideWgs : 512) + BH - 1) / BH;
    const int ns_max = cfg.values_on_host ? sd::kDecodeMaxSplits : sd::kDecodeWideSplits;
    ns = ns < 1 ? 1 : ns > ns_max ? ns_max : ns;
    const int cap = (c->max_blocks + 3) / 4;
    c->nsplit = ns > cap ? cap : ns;
    // device values: split the splits between sink/window blocks and kept
    // blocks, a sink/window split taking about 1.25 times the blocks of a
    // kept-block split, which starts only after its selects (14 of 48 at
    // these shapes; 10 and 12 measured slower)
    const int64_t ra = (cfg.sink > 0 || cfg.window > 0) ? (cfg.sink + 7) / 8 + (cfg.window + 7) / 8 + 1 : 0;
    const int64_t rk = int64_t(last.keep) * (last.chunk / 8);
    if (cfg.values_on_host || ra == 0) {
        c->nsplit_a = 0;
    } else {
        if (c->nsplit < 2) c->nsplit = 2;
        const int64_t den = 4 * ra + 5 * rk;
        int na = int((int64_t(c->nsplit) * 4 * ra + den / 2) / den);
        na = na < 1 ? 1 : na > c->nsplit - 1 ? c->nsplit - 1 : na;
        c->nsplit_a = na;
    }
    // Fuse the last stage Q into the kernel of the stage P before it.
    // Possible when Q's chunks are exactly 8 sampled rows (one load slot),
    // Q's stride divides P's (so P's samples are among the rows read), P
    // reads at most 4x its own samples, all children's scores fit in LDS,
    // and Q's select keeps its keys in registers (at most 512 candidates).
    // (With host values the value-cache kernel takes the two selects.)  It
    // trades one kernel boundary and one scoring pass for a second select
    // in the decode kernel and more rows read by P: P reads
    // every row at Q's stride of each of its candidates instead of its own
    // samples, while an unfused Q kernel reads Q.ncand x 8 rows.  Fused when
    // those extra bytes over all (request, KV head) pipelines stay within
    // kFuseExtraBytes, about 1.6 us of streaming: then the saved boundary
    // and scoring pass (about 2 us, measured) win; with many requests in
    // flight the step is bandwidth-bound and the extra rows cost more (16
    // requests of up to 128K: 139 us unfused against 148 us fused; 1 request:
    // 36.5 against 38.5 us at 128K, 55.7 against 58.1 us at 1M).
    // SD_FUSE_LAST_STAGE=0 never fuses, =1 fuses whenever possible.
    constexpr int64_t kFuseExtraBytes = int64_t(8) << 20;
    c->fuse = 0;
    c->fuse_rq = 0;
    c->fuse_m = 0;
    const char* fenv = std::getenv("SD_FUSE_LAST_STAGE");
    const int fuse_mode = !fenv ? -1 : fenv[0] == '0' ? 0 : 1;     // -1: by the extra bytes
    if (fuse_mode != 0 && cfg.num_stages >= 2) {
        sd::StageGeom& P = c->st[cfg.num_stages - 2];
        const sd::StageGeom& Q = c->st[cfg.num_stages - 1];
        const int rq = P.chunk / Q.chunk;
        const int64_t extra_rows = int64_t(P.ncand) * (P.chunk / Q.stride - P.chunk / P.stride) -
                                   int64_t(Q.ncand) * (Q.chunk / Q.stride);
        const bool worth = fuse_mode == 1 || int64_t(BH) * extra_rows * sd::kHeadDim <= kFuseExtraBytes;
        if (worth && Q.chunk / Q.stride == 8 && P.stride % Q.stride == 0 && P.stride / Q.stride <= 4 &&
            P.chunk / Q.stride <= kMaxSamples && int64_t(P.ncand) * rq <= 8192 && Q.ncand <= 512) {
            c->fuse = 1;
            c->fuse_rq = rq;
            c->fuse_m = P.stride / Q.stride;
            P.nrows = P.chunk / Q.stride;
            P.rstride = Q.stride;
            const int ns8 = (P.nrows + 7) / 8;
            const int ns8p = ns8 == 1 ? 1 : ns8 == 2 ? 2 : ns8 <= 4 ? 4 : 8;
            P.per_wg = 4 * (ns8p >= 8 ? 1 : 8 / ns8p);
            P.nwg = (P.ncand + P.per_wg - 1) / P.per_wg;
        }
    }
    // Unfused, with stage S-2's stride twice stage S-1's and 8 rows per
    // stage S-1 chunk, and many pipelines: stage S-2 also stores each
    // child's maximum over the 4 of its 8 rows it reads anyway, and stage
    // S-1 reads only the other 4 (half its bytes; the score is the larger
    // maximum, exactly).  16 requests of up to 128K: stage 2 16.3 -> 12.0 us,
    // the step 125.8 -> 122.3 us.  With few pipelines the stages are
    // latency, not bytes, and stage S-1's 16 candidates per wave halve its
    // workgroups: one request unfused, 35.7 -> 36.5 us at 128K.
    // SD_HALF_ROWS=0 reads every row in stage S-1.
    c->half = 0;
    c->half_rq = 0;
    const char* henv = std::getenv("SD_HALF_ROWS");
    if (!c->fuse && cfg.num_stages >= 2 && BH >= sd::kDecodeWideMinPipes && !(henv && henv[0] == '0')) {
        const sd::StageGeom& P = c->st[cfg.num_stages - 2];
        const sd::StageGeom& Q = c->st[cfg.num_stages - 1];
        const int rq = P.chunk / Q.chunk;
        // (rq a power of two from 2 to 16: stage S-2 reads 4 rq rows, whole
        // 8-row load slots of 2 children each, in an instantiated slot count)
        if (Q.chunk / Q.stride == 8 && P.stride == 2 * Q.stride && P.chunk % Q.chunk == 0 && rq >= 2 &&
            (rq & (rq - 1)) == 0 && rq <= 16) {
            c->half = 1;
            c->half_rq = P.chunk / Q.chunk;
        }
    }
    // With many pipelines the unfused stages after the first score two load
    // batches per wave: half the workgroups, so half the redundant selects
    // at their heads (16 requests of up to 128K: stage 1 26.3 -> 24.7 us).
    if (BH >= sd::kDecodeWideMinPipes) {
        for (int s = 1; s < cfg.num_stages; ++s) {
            sd::StageGeom& g = c->st[s];
            if (c->fuse && s == cfg.num_stages - 2) continue;
            const int cpw = 2 * (g.per_wg / 4);
            if (cpw > sd::kMaxCandPerWave) continue;
            g.per_wg = 4 * cpw;
            g.nwg = (g.ncand + g.per_wg - 1) / g.per_wg;
        }
    }
    // (stage S-2's row scores are staged per wave in LDS: 256 words, 128
    // with every geometry above; checked, not assumed)
    if (c->half && (c->st[cfg.num_stages - 2].per_wg / 4) * c->st[cfg.num_stages - 2].nrows > 256) c->half = 0;
    const float scale = cfg.softmax_scale > 0.0f ? cfg.softmax_scale : 1.0f / std::sqrt(float(cfg.head_dim));
    c->scale_log2 = scale * 1.4426950408889634f;

    if (cfg.values_on_host) {
        if (cfg.value_cache_tokens < 8 || cfg.value_cache_tokens % 8 != 0) return SD_ERR_INVALID_ARG;
        if (cfg.value_cache_tokens / 8 < c->max_blocks) return SD_ERR_INVALID_ARG;
        if (cfg.value_cache_tokens / 8 > (int64_t(1) << 24)) return SD_ERR_UNSUPPORTED;
    }
    // the LRU step on chip for small caches; SD_VCACHE_ONCHIP=0 takes the
    // device-memory path for every size
    const char* venv = std::getenv("SD_VCACHE_ONCHIP");
    c->vc_onchip = cfg.values_on_host && cfg.value_cache_tokens / 8 <= sd::kVcOnchipSlots &&
                   c->max_blocks <= sd::kVcOnchipBlocks && !(venv && venv[0] == '0');
    return SD_OK;
}

// Runs one launch, handing it a pair of profiling events (carried by the
// dispatch itself) when its kind is being timed.
template <class F>
hipError_t timed(sd_ctx* c, int kind, hipStream_t s, F&& launch_fn) {
    (void)s;
    const bool on = c->prof_ev && ((c->prof_mask >> kind) & 1u) && c->prof_n < c->prof_max;
    if (!on) return launch_fn(sd::Timing{});
    sd::Timing t{c->prof_ev[2 * c->prof_n], c->prof_ev[2 * c->prof_n + 1]};
    const hipError_t e = launch_fn(t);
    if (e == hipSuccess) {
        c->prof_kind[c->prof_n] = int8_t(kind);
        ++c->prof_n;
    }
    return e;
}

void free_profiler(sd_ctx* c) {
    if (c->prof_ev) {
        for (int i = 0; i < 2 * c->prof_max; ++i)
            if (c->prof_ev[i]) (void)hipEventDestroy(c->prof_ev[i]);
        delete[] c->prof_ev;
        delete[] c->prof_kind;
    }
    c->prof_ev = nullptr;
    c->prof_kind = nullptr;
    c->prof_max = c->prof_n = 0;
    c->prof_mask = 0;
}

struct Carver {
    size_t off = 0;
    template <class T>
    size_t take(size_t count) {
        size_t o = off;
        off = round_up(off + count * sizeof(T), 256);
        return o;
    }
};

// Device-dependent part of a context's set-up (no allocation): the device,
// the LDS check of the largest kernel, and the dense decode's split count.
sd_status device_setup(sd_ctx* c) {
    hipError_t e0 = hipGetDevice(&c->device);
    if (e0 != hipSuccess) return from_hip(e0, "hipGetDevice");
    int lds_max = 0;
    e0 = hipDeviceGetAttribute(&lds_max, hipDeviceAttributeMaxSharedMemoryPerBlock, c->device);
    if (e0 != hipSuccess) return from_hip(e0, "hipDeviceGetAttribute");
    // stage s's select runs at the head of stage s + 1's pruning kernel,
    // the last stage's (fused: the last two stages') at the head of the
    // decode kernel.  The pruning kernels' static LDS is the query codes,
    // the exchange words and the candidate starts (4 waves x kMaxCandPerWave); the decode
    // kernel's is the four waves' softmax state (m, l and the G x 128
    // accumulators), the exchange words, the block tile's starts and masks,
    // the hand-off word and the merge's reduction (one float4 per thread).
    const int64_t prune_static = 4 * (sd::kHeadDim + 32 + 4 * sd::kMaxCandPerWave);
    const int64_t attend_static = 4 * (4 * (2 + sd::kHeadDim) * int64_t(c->G) + 32 + 2 * 256 + 1 + 4 * 256);
    int64_t need = 0;
    for (int s = 0; s + 1 < c->S; ++s)
        need = std::max<int64_t>(need, 4 * int64_t(sd::kept_lds_words(sd::stage_dev(c, s), s == 0)) + prune_static);
    const int64_t last_words = c->fuse ? sd::fused_lds_words(sd::stage_dev(c, c->S - 2), c->S == 2,
                                                             sd::stage_dev(c, c->S - 1), c->fuse_rq)
                                       : sd::kept_lds_words(sd::stage_dev(c, c->S - 1), c->S == 1);
    need = std::max(need, 4 * last_words + attend_static);
    // half: stage S-1's kernel keeps stage S-2's kept indices too, and the
    // stored-maximum index of each of its candidates
    // and stage S-2's kernel stages its row scores (4 waves x 320 words)
    if (c->half) {
        need = std::max<int64_t>(need, 4 * int64_t(sd::kept_lds_words(sd::stage_dev(c, c->S - 2), c->S == 2) +
                                                    c->st[c->S - 2].keep) +
                                           prune_static + 4 * 4 * 16);
        need = std::max<int64_t>(
            need, (c->S >= 3 ? 4 * int64_t(sd::kept_lds_words(sd::stage_dev(c, c->S - 3), c->S == 3)) : 0) +
                      prune_static + 4 * 4 * (256 + 64));
    }
    // (unfused with the stage before the last reused, the last stage is selected in the decode kernel too)
    need = std::max(need, 4 * int64_t(sd::kept_lds_words(sd::stage_dev(c, c->S - 1), c->S == 1)) + attend_static);
    if (c->cfg.values_on_host) {
        // the value-cache kernel takes the selects instead, next to its LRU
        // state (on chip: the touched map, the block list, the evicted
        // slots and the padded recency order)
        const int64_t vcache_static =
            4 * (32 + (c->vc_onchip ? int64_t(sd::kVcOnchipSlots / 32 + 2 * sd::kVcOnchipBlocks + sd::kVcOnchipSlots +
                                              sd::kVcOnchipSlots / 32)
                                    : 3));
        need = std::max(need, 4 * last_words + vcache_static);
        need = std::max(need, 4 * int64_t(sd::kept_lds_words(sd::stage_dev(c, c->S - 1), c->S == 1)) + vcache_static);
    }
    if (need > lds_max) {
        std::snprintf(g_last_error, sizeof(g_last_error), "a kernel needs %lld bytes of LDS, more than the %d a "
                      "workgroup has", (long long)need, lds_max);
        return SD_ERR_UNSUPPORTED;
    }
    // Dense decode (sd_dense_decode): 8 workgroups per compute unit in
    // all (about 2.7 times the kernel's resident occupancy of 3, which
    // measured faster than one resident wave of workgroups at 128K and
    // 1M; SD_DENSE_WG_PER_CU overrides the 8), at most 512 splits per
    // (request, KV head) (the merge's limit), at least 32 blocks of the
    // longest request per split.
    int cus = 0, occ = 8;
    e0 = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, c->device);
    if (e0 != hipSuccess) return from_hip(e0, "hipDeviceGetAttribute");
    if (const char* env = std::getenv("SD_DENSE_WG_PER_CU")) {
        const int o = std::atoi(env);
        if (o >= 1 && o <= 64) occ = o;
    }
    const int64_t BH = int64_t(c->cfg.batch) * c->cfg.num_kv_heads;
    const int64_t nbmax = (c->cfg.max_context + 7) / 8;
    int64_t nd = (int64_t(std::max(cus, 1)) * std::max(occ, 1) + BH - 1) / BH;
    nd = std::min<int64_t>(nd, 512);
    nd = std::min<int64_t>(nd, std::max<int64_t>(1, (nbmax + 31) / 32));
    c->nsplit_d = int(std::max<int64_t>(nd, 1));
    return SD_OK;
}

// Workspace layout of a planned context, every region 256-byte aligned.
// Returns the bytes it needs; when base is not null, also points the
// context's workspace members into [base, base + bytes).  dense: room for
// the dense decode's split partials as well (sd_dense_decode).
size_t carve_workspace(sd_ctx* c, char* base, bool dense) {
    const size_t BH = size_t(c->cfg.batch) * size_t(c->cfg.num_kv_heads);
    Carver cv;
    // the hand-off counters first, the error flag right after them: one
    // contiguous run that sd_decode_step_noalloc clears with one fill
    const size_t o_tick = cv.take<int32_t>(BH * sd::kTickInts);
    const size_t o_flag = cv.take<int32_t>(1);
    size_t o_scores[SD_MAX_STAGES];
    for (int s = 0; s < c->S; ++s) o_scores[s] = cv.take<int32_t>(BH * c->st[s].ncand);
    const size_t o_qg = cv.take<int32_t>(BH * sd::kHeadDim);
    const size_t o_blocks = cv.take<uint32_t>(BH * c->max_blocks);
    const size_t o_nblocks = cv.take<int32_t>(BH);
    const size_t nsp = size_t(dense ? std::max(c->nsplit, c->nsplit_d) : c->nsplit);
    const size_t o_part = cv.take<float>(BH * nsp * c->G * (2 + sd::kHeadDim));
    const size_t o_abs = cv.take<unsigned>(BH);
    const size_t o_req = cv.take<int32_t>(BH);
    const size_t o_pre = c->fuse   ? cv.take<int32_t>(BH * size_t(c->st[c->S - 2].ncand) * c->fuse_rq)
                         : c->half ? cv.take<int32_t>(BH * size_t(c->st[c->S - 2].ncand) * c->half_rq)
                                   : 0;
    size_t o_vc[11] = {0};
    if (c->cfg.values_on_host) {
        c->vc.slots = int32_t(c->cfg.value_cache_tokens / 8);
        c->vc.nblk_max = int32_t((c->Lmax + 7) / 8);
        o_vc[0] = cv.take<uint16_t>(BH * size_t(c->vc.slots) * 8 * sd::kHeadDim);
        o_vc[1] = cv.take<int32_t>(BH * size_t(c->vc.nblk_max));
        o_vc[2] = cv.take<int32_t>(BH * size_t(c->vc.slots));
        o_vc[3] = cv.take<int32_t>(BH * size_t(c->vc.slots));
        o_vc[4] = cv.take<int32_t>(BH);
        o_vc[5] = cv.take<int32_t>(2 * BH * size_t(c->vc.slots));
        o_vc[6] = cv.take<int32_t>(BH * size_t(c->max_blocks));
        o_vc[7] = cv.take<int32_t>(BH * size_t(c->max_blocks));
        o_vc[8] = cv.take<int64_t>(sd::kVcCounters);
        o_vc[9] = cv.take<int32_t>(BH * size_t(c->vc.slots));
        o_vc[10] = cv.take<int32_t>(BH);
    }
    if (!base) return cv.off;
    for (int s = 0; s < c->S; ++s) c->scores[s] = reinterpret_cast<int32_t*>(base + o_scores[s]);
    c->qgroup = reinterpret_cast<int32_t*>(base + o_qg);
    c->blocks = reinterpret_cast<uint32_t*>(base + o_blocks);
    c->nblocks = reinterpret_cast<int32_t*>(base + o_nblocks);
    c->part = reinterpret_cast<float*>(base + o_part);
    c->absmax_bits = reinterpret_cast<unsigned*>(base + o_abs);
    c->requant = reinterpret_cast<int32_t*>(base + o_req);
    c->tick = reinterpret_cast<int32_t*>(base + o_tick);
    c->flag = reinterpret_cast<int32_t*>(base + o_flag);
    c->pre = c->fuse || c->half ? reinterpret_cast<int32_t*>(base + o_pre) : nullptr;
    if (c->cfg.values_on_host) {
        c->vc.pool = reinterpret_cast<uint16_t*>(base + o_vc[0]);
        c->vc.page = reinterpret_cast<int32_t*>(base + o_vc[1]);
        c->vc.slot_block = reinterpret_cast<int32_t*>(base + o_vc[2]);
        c->vc.slot_last = reinterpret_cast<int32_t*>(base + o_vc[3]);
        c->vc.used = reinterpret_cast<int32_t*>(base + o_vc[4]);
        c->vc.order = reinterpret_cast<int32_t*>(base + o_vc[5]);
        c->vc.evicted = reinterpret_cast<int32_t*>(base + o_vc[6]);
        c->vc.blk_slot = reinterpret_cast<int32_t*>(base + o_vc[7]);
        c->vc.counters = reinterpret_cast<int64_t*>(base + o_vc[8]);
        c->vc.slot_fill = reinterpret_cast<int32_t*>(base + o_vc[9]);
        c->vc.stepc = reinterpret_cast<int32_t*>(base + o_vc[10]);
    }
    return cv.off;
}

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxScratchDevices];     // device address of `scratch` on each GPU, null until looked up

// Address of the scratch array on device `dev` (which must be current),
// looked up on the first call for that device.
sd_status scratch_on_device(int dev, void** out) {
    if (dev < 0 || dev >= kMaxScratchDevices) {
        std::snprintf(g_last_error, sizeof(g_last_error), "device %d: no scratch slot (at most %d devices)", dev,
                      kMaxScratchDevices);
        return SD_ERR_UNSUPPORTED;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void* ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return from_hip(e, "hipGetSymbolAddress(scratch)");
        if (!ptr) return from_hip(hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
        g_scratch_dev[dev] = ptr;
    }
    *out = g_scratch_dev[dev];
    return SD_OK;
}

// Zeroes n words (a fill kernel rather than a memset, so that a caller may
// capture the call in a graph).
__global__ void sd_clear_words_kernel(int32_t* p, int n) {
    const int i = int(blockIdx.x * blockDim.x + threadIdx.x);
    if (i < n) p[i] = 0;
}

}  // namespace

extern "C" {

const char* sd_last_error(void) { return g_last_error; }

const char* sd_status_string(sd_status s) {
    switch (s) {
        case SD_OK: return "ok";
        case SD_ERR_INVALID_ARG: return "invalid argument";
        case SD_ERR_UNSUPPORTED: return "unsupported configuration";
        case SD_ERR_OUT_OF_MEMORY: return "out of device memory";
        case SD_ERR_HIP: return "HIP runtime error";
        case SD_ERR_DEVICE_FLAG: return "device flagged bad input (length outside [1, max_context])";
    }
    return "unknown status";
}

sd_status sd_create(const sd_config* cfg, sd_ctx** out) {
    if (!out) return SD_ERR_INVALID_ARG;
    *out = nullptr;
    if (!cfg) return SD_ERR_INVALID_ARG;
    sd_ctx* c = new (std::nothrow) sd_ctx();
    if (!c) return SD_ERR_OUT_OF_MEMORY;
    sd_status st = plan(*cfg, c);
    if (st == SD_OK) st = device_setup(c);
    if (st != SD_OK) { delete c; return st; }
    c->ws_bytes = carve_workspace(c, nullptr, true);
    hipError_t e = hipMalloc(&c->ws, c->ws_bytes);
    if (e != hipSuccess) { (void)hipGetLastError(); delete c; return from_hip(e, "hipMalloc(workspace)"); }
    carve_workspace(c, static_cast<char*>(c->ws), true);
    // Flag and score buffers start defined; this is setup, outside any step.
    e = hipMemset(c->ws, 0, c->ws_bytes);
    if (e == hipSuccess && cfg->values_on_host) e = sd::launch_value_cache_reset(c, nullptr);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) { (void)hipFree(c->ws); delete c; return from_hip(e, "workspace initialisation"); }
    *out = c;
    return SD_OK;
}

void sd_destroy(sd_ctx* c) {
    if (!c) return;
    int cur = -1;
    (void)hipGetDevice(&cur);
    if (cur != c->device) (void)hipSetDevice(c->device);
    (void)hipDeviceSynchronize();
    free_profiler(c);
    if (c->vside) (void)hipStreamDestroy(c->vside);
    if (c->vside_done) (void)hipEventDestroy(c->vside_done);
    if (c->vstage) (void)hipHostFree(c->vstage);
    (void)hipFree(c->ws);
    if (cur != c->device && cur >= 0) (void)hipSetDevice(cur);
    delete c;
}

sd_status sd_quantize_keys(sd_ctx* c, const uint16_t* k, const int32_t* lengths, int8_t* k8, float* absmax,
                           void* stream) {
    if (!c || !k || !lengths || !k8) return SD_ERR_INVALID_ARG;
    if (!aligned16(k) || !aligned16(k8)) return SD_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    return from_hip(timed(c, SD_PROF_QUANTIZE, s,
                          [&](sd::Timing t) { return sd::launch_quantize_keys(c, k, lengths, k8, absmax, s, t); }));
}

sd_status sd_append_kv(sd_ctx* c, const uint16_t* k_new, const uint16_t* v_new, int32_t n_new, const int32_t* lengths,
                       uint16_t* k, int8_t* k8, uint16_t* v, uint8_t* k4, float* absmax, void* stream) {
    if (!c || !k_new || !v_new || !lengths || !k || !k8 || !v) return SD_ERR_INVALID_ARG;
    if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k) || !aligned16(k8) || !aligned16(v) ||
        (k4 && !aligned16(k4)))
        return SD_ERR_INVALID_ARG;
    if (n_new < 1 || n_new > c->Lmax) return SD_ERR_INVALID_ARG;
    if (c->cfg.values_on_host) return SD_ERR_UNSUPPORTED;
    hipStream_t s = static_cast<hipStream_t>(stream);
    return from_hip(timed(c, SD_PROF_APPEND, s, [&](sd::Timing t) {
        return sd::launch_append(c, k_new, v_new, n_new, lengths, k, k8, v, k4, absmax, s, t);
    }));
}

sd_status sd_quantize_query(sd_ctx* c, const uint16_t* q, int8_t* q8, int32_t* qg, void* stream) {
    if (!c || !q) return SD_ERR_INVALID_ARG;
    if (!aligned16(q)) return SD_ERR_INVALID_ARG;
    return from_hip(sd::launch_quantize_query(c, q, q8, qg, static_cast<hipStream_t>(stream)));
}

namespace {

// SD_VALUE_FETCH_COPY, after the value-cache kernel of a step on stream s:
// waits for the step's attended block list, then copies every missed (or
// refilled) block's rows t < L from host memory v into its slot, one
// hipMemcpyAsync per run of blocks consecutive both in host memory and in
// the slot pool, on the side stream; s waits for them before the decode
// kernel.
hipError_t copy_missed_blocks(sd_ctx* c, const uint16_t* v, const int32_t* lengths, hipStream_t s) {
    const int B = c->cfg.batch, Hkv = c->cfg.num_kv_heads, BH = B * Hkv, MB = c->max_blocks;
    int32_t* h_nb = c->vstage;
    int32_t* h_len = h_nb + BH;
    int32_t* h_blocks = h_len + B;
    int32_t* h_slot = h_blocks + int64_t(BH) * MB;
    hipError_t e = hipMemcpyAsync(h_nb, c->nblocks, sizeof(int32_t) * BH, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipMemcpyAsync(h_len, lengths, sizeof(int32_t) * B, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess)
        e = hipMemcpyAsync(h_blocks, c->blocks, sizeof(int32_t) * BH * MB, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess)
        e = hipMemcpyAsync(h_slot, c->vc.blk_slot, sizeof(int32_t) * BH * MB, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return e;
    constexpr int64_t kBlockElems = 8 * sd::kHeadDim;
    const int64_t slots = c->vc.slots;
    int64_t runs = 0;
    for (int bj = 0; bj < BH && e == hipSuccess; ++bj) {
        const int64_t L = h_len[bj / Hkv];
        if (L < 1 || L > c->Lmax) continue;          // no blocks (flagged by the pruning kernels)
        const int nb = std::min(h_nb[bj], MB);
        int64_t run_blk = -1, run_slot = -1, run_rows = 0;
        auto flush = [&]() -> hipError_t {
            if (run_rows == 0) return hipSuccess;
            ++runs;
            return hipMemcpyAsync(c->vc.pool + (int64_t(bj) * slots + run_slot) * kBlockElems,
                                  v + (int64_t(bj) * c->Lmax + run_blk * 8) * sd::kHeadDim,
                                  size_t(run_rows) * sd::kHeadDim * sizeof(uint16_t), hipMemcpyHostToDevice,
                                  c->vside);
        };
        for (int r = 0; r < nb && e == hipSuccess; ++r) {
            const int32_t se = h_slot[int64_t(bj) * MB + r];
            if (!(se & (sd::kVcMissBit | sd::kVcRefillBit))) continue;
            const int64_t blk = int64_t(uint32_t(h_blocks[int64_t(bj) * MB + r]) >> 8);
            const int64_t slot = se & sd::kVcSlotMask;
            const int64_t rows = std::min<int64_t>(8, L - 8 * blk);
            if (rows <= 0 || slot >= slots) continue;
            // extends the run when both sides continue it (the run's rows so far are whole blocks)
            if (run_rows > 0 && run_rows % 8 == 0 && blk == run_blk + run_rows / 8 && slot == run_slot + run_rows / 8) {
                run_rows += rows;
                continue;
            }
            e = flush();
            run_blk = blk;
            run_slot = slot;
            run_rows = rows;
        }
        if (e == hipSuccess) e = flush();
    }
    c->vcopies = runs;
    if (e == hipSuccess) e = hipEventRecord(c->vside_done, c->vside);
    if (e == hipSuccess) e = hipStreamWaitEvent(s, c->vside_done, 0);
    return e;
}

// One decode step; k4 (the int4 first-stage sketch) or null.
sd_status decode_step(sd_ctx* c, const uint16_t* q, const uint16_t* k, const int8_t* k8, const uint8_t* k4,
                      const uint16_t* v, const int32_t* lengths, uint16_t* out, int32_t* kept, int32_t reuse,
                      void* stream) {
    if (!c || !q || !k || !k8 || !v || !lengths || !out || !kept) return SD_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(k8) || !aligned16(v) || !aligned16(out))
        return SD_ERR_INVALID_ARG;
    if (reuse < 0 || reuse > c->S) return SD_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool vcopy = c->cfg.values_on_host && c->vfetch == SD_VALUE_FETCH_COPY;
    if (vcopy) {
        // the copies wait for the host, which a captured graph cannot do
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(s, &cs) != hipSuccess) return from_hip(hipGetLastError());
        if (cs != hipStreamCaptureStatusNone) return SD_ERR_UNSUPPORTED;
    }
    const uint16_t* vk = v;
    if (c->cfg.values_on_host) {
        // v is pinned host memory: the kernels read it through its device alias
        if (v != c->vhost_key) {
            void* dev = nullptr;
            if (hipHostGetDevicePointer(&dev, const_cast<uint16_t*>(v), 0) != hipSuccess || !dev) {
                (void)hipGetLastError();
                return SD_ERR_INVALID_ARG;
            }
            c->vhost_key = v;
            c->vhost_dev = static_cast<const uint16_t*>(dev);
        }
        vk = c->vhost_dev;
    }
    hipError_t e = hipSuccess;
    // Stages [0, reuse) keep the kept sets that kept_idx holds; the first
    // stage run reads its parents from there.  The fused plan (the last
    // stage scored inside the kernel of the one before, both selected by
    // the decode kernel) serves while that stage before the last runs;
    // when it is reused, the last stage runs in a kernel of its own.  The
    // decode kernel's last split per (request, KV head) writes the output.
    const bool fused = c->fuse && reuse <= c->S - 2;
    const int nprune = fused ? c->S - 1 : c->S;
    for (int st = reuse; st < nprune && e == hipSuccess; ++st)
        e = timed(c, SD_PROF_STAGE0 + st, s, [&](sd::Timing t) {
            return sd::launch_prune_stage(c, st, st == reuse && st > 0, fused, q, k8, k4, lengths, kept, s, t);
        });
    const bool last_given = reuse == c->S;
    if (e == hipSuccess && c->cfg.values_on_host)
        e = timed(c, SD_PROF_VALUE_CACHE, s, [&](sd::Timing t) {
            return sd::launch_value_cache_update(c, last_given, fused, lengths, kept, s, t);
        });
    if (e == hipSuccess && vcopy) e = copy_missed_blocks(c, v, lengths, s);
    if (e == hipSuccess)
        e = timed(c, SD_PROF_ATTEND, s, [&](sd::Timing t) {
            return sd::launch_attend(c, last_given, fused, q, k, vk, lengths, kept, out, s, t);
        });
    return from_hip(e);
}

sd_status sd_dense_decode(sd_ctx* c, const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* lengths,
                          uint16_t* out, void* stream) {
    if (!c || !q || !k || !v || !lengths || !out) return SD_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return SD_ERR_INVALID_ARG;
    if (c->cfg.values_on_host) return SD_ERR_UNSUPPORTED;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = timed(c, SD_PROF_DENSE, s,
                         [&](sd::Timing t) { return sd::launch_dense(c, q, k, v, lengths, s, t); });
    if (e == hipSuccess)
        e = timed(c, SD_PROF_COMBINE, s,
                  [&](sd::Timing t) { return sd::launch_combine(c, c->nsplit_d, out, s, t); });
    return from_hip(e);
}

}  // namespace

sd_status sd_decode_step_reuse(sd_ctx* c, const uint16_t* q, const uint16_t* k, const int8_t* k8, const uint16_t* v,
                               const int32_t* lengths, uint16_t* out, int32_t* kept, int32_t reuse, void* stream) {
    return decode_step(c, q, k, k8, nullptr, v, lengths, out, kept, reuse, stream);
}

sd_status sd_decode_step(sd_ctx* c, const uint16_t* q, const uint16_t* k, const int8_t* k8, const uint16_t* v,
                         const int32_t* lengths, uint16_t* out, int32_t* kept, void* stream) {
    return decode_step(c, q, k, k8, nullptr, v, lengths, out, kept, 0, stream);
}

sd_status sd_decode_step_noalloc(const sd_config* cfg, const uint16_t* q, const uint16_t* k, const int8_t* k8,
                                 const uint16_t* v, const int32_t* lengths, uint16_t* out, int32_t* kept,
                                 void* stream) {
    if (!cfg) return SD_ERR_INVALID_ARG;
    if (cfg->values_on_host) {
        std::snprintf(g_last_error, sizeof(g_last_error), "sd_decode_step_noalloc: values in host memory need a "
                      "context (sd_create) for their value cache");
        return SD_ERR_UNSUPPORTED;
    }
    sd_ctx c{};                  // the plan, on the stack; its workspace is the scratch array
    sd_status st = plan(*cfg, &c);
    if (st == SD_OK) st = device_setup(&c);
    if (st != SD_OK) return st;
    const size_t need = carve_workspace(&c, nullptr, false);
    if (need > kNoAllocScratchBytes) {
        std::snprintf(g_last_error, sizeof(g_last_error), "sd_decode_step_noalloc: the step needs %zu bytes of "
                      "workspace, more than the %zu of the scratch array", need, kNoAllocScratchBytes);
        return SD_ERR_UNSUPPORTED;
    }
    void* base = nullptr;
    st = scratch_on_device(c.device, &base);
    if (st != SD_OK) return st;
    carve_workspace(&c, static_cast<char*>(base), false);
    c.ws = base;
    c.ws_bytes = need;
    // the scratch keeps the last call's contents, possibly of another
    // configuration: the hand-off counters and the error flag (one run at
    // the start of the workspace) must start at zero; every other word a
    // step reads, it writes first
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int nclear = int((c.flag - c.tick) + 1);
    sd_clear_words_kernel<<<(nclear + 255) / 256, 256, 0, s>>>(c.tick, nclear);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return from_hip(e, "sd_clear_words_kernel");
    return decode_step(&c, q, k, k8, nullptr, v, lengths, out, kept, 0, stream);
}

int64_t sd_sketch4_rows(const sd_ctx* c) { return c ? c->sketch_rows : -1; }

sd_status sd_quantize_sketch4(sd_ctx* c, const uint16_t* k, const int32_t* lengths, uint8_t* k4, void* stream) {
    if (!c || !k || !lengths || !k4) return SD_ERR_INVALID_ARG;
    if (!aligned16(k) || !aligned16(k4)) return SD_ERR_INVALID_ARG;
    return from_hip(sd::launch_sketch4(c, k, lengths, k4, static_cast<hipStream_t>(stream)));
}

sd_status sd_decode_step_sketch4(sd_ctx* c, const uint16_t* q, const uint16_t* k, const int8_t* k8,
                                 const uint8_t* k4, const uint16_t* v, const int32_t* lengths, uint16_t* out,
                                 int32_t* kept, void* stream) {
    if (!c || !k4) return SD_ERR_INVALID_ARG;
    if (!aligned16(k4)) return SD_ERR_INVALID_ARG;
    // the first stage must run in a kernel of its own (not fused with the
    // last stage, which reads rows the sketch does not hold)
    if (c->fuse && c->S == 2) return SD_ERR_UNSUPPORTED;
    return decode_step(c, q, k, k8, k4, v, lengths, out, kept, 0, stream);
}

int64_t sd_stage_candidates(const sd_ctx* c, int32_t stage) {
    if (!c || stage < 0 || stage >= c->S) return -1;
    return c->st[stage].ncand;
}

sd_status sd_set_value_fetch(sd_ctx* c, int32_t mode) {
    if (!c) return SD_ERR_INVALID_ARG;
    if (mode != SD_VALUE_FETCH_MAPPED && mode != SD_VALUE_FETCH_COPY) return SD_ERR_INVALID_ARG;
    if (!c->cfg.values_on_host) return SD_ERR_UNSUPPORTED;
    if (mode == SD_VALUE_FETCH_COPY && !c->vstage) {
        int cur = -1;
        (void)hipGetDevice(&cur);
        if (cur != c->device) (void)hipSetDevice(c->device);
        const int64_t BH = int64_t(c->cfg.batch) * c->cfg.num_kv_heads;
        const size_t bytes = sizeof(int32_t) * size_t(BH + c->cfg.batch + 2 * BH * c->max_blocks);
        hipError_t e = hipStreamCreateWithFlags(&c->vside, hipStreamNonBlocking);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&c->vside_done, hipEventDisableTiming);
        void* h = nullptr;
        if (e == hipSuccess) e = hipHostMalloc(&h, bytes, hipHostMallocDefault);
        if (cur != c->device && cur >= 0) (void)hipSetDevice(cur);
        if (e != hipSuccess) {
            if (c->vside) (void)hipStreamDestroy(c->vside);
            if (c->vside_done) (void)hipEventDestroy(c->vside_done);
            c->vside = nullptr;
            c->vside_done = nullptr;
            return from_hip(e, "sd_set_value_fetch");
        }
        c->vstage = static_cast<int32_t*>(h);
    }
    c->vfetch = mode;
    return SD_OK;
}

sd_status sd_record_attended(sd_ctx* c, uint32_t* dst, int64_t dst_len) {
    if (!c) return SD_ERR_INVALID_ARG;
    if (!dst) {
        c->rec = nullptr;
        return SD_OK;
    }
    if (dst_len < int64_t(c->cfg.batch) * c->cfg.num_kv_heads * c->max_blocks) return SD_ERR_INVALID_ARG;
    if (c->Lmax > (int64_t(1) << 27)) return SD_ERR_UNSUPPORTED;    // block ids must fit 24 bits
    c->rec = dst;
    return SD_OK;
}

sd_status sd_stage_scores(sd_ctx* c, int32_t stage, int32_t* dst, int64_t dst_len, void* stream) {
    if (!c || !dst || stage < 0 || stage >= c->S) return SD_ERR_INVALID_ARG;
    const int64_t n = int64_t(c->cfg.batch) * c->cfg.num_kv_heads * c->st[stage].ncand;
    if (dst_len < n) return SD_ERR_INVALID_ARG;
    return from_hip(hipMemcpyAsync(dst, c->scores[stage], size_t(n) * 4, hipMemcpyDeviceToDevice,
                                   static_cast<hipStream_t>(stream)));
}

sd_status sd_check(sd_ctx* c, void* stream) {
    if (!c) return SD_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipStreamSynchronize(s);
    if (e != hipSuccess) return from_hip(e);
    int32_t flag = 0;
    e = hipMemcpy(&flag, c->flag, sizeof(flag), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return from_hip(e);
    if (flag) {
        e = hipMemset(c->flag, 0, sizeof(int32_t));
        if (e != hipSuccess) return from_hip(e);
        std::snprintf(g_last_error, sizeof(g_last_error), "%s%s",
                      (flag & sd::kFlagBadLength) ? "a length outside [1, max_context]; " : "",
                      (flag & sd::kFlagPlacement) ? "the workgroups of one (request, KV head) ran on more than one "
                                                    "XCD: their hand-offs, and the results, are not reliable" : "");
        return SD_ERR_DEVICE_FLAG;
    }
    return SD_OK;
}

sd_status sd_get_stats(sd_ctx* c, sd_stats* out, void* stream) {
    if (!c || !out) return SD_ERR_INVALID_ARG;
    std::memset(out, 0, sizeof(*out));
    hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return from_hip(e);
    if (!c->cfg.values_on_host) return SD_OK;
    int64_t h[sd::kVcCounters];
    e = hipMemcpy(h, c->vc.counters, sizeof(h), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return from_hip(e);
    out->steps = h[0];
    out->blocks_needed = h[1];
    out->hits = h[2];
    out->misses = h[3];
    out->refills = h[12];
    out->h2d_bytes = (h[3] + h[12]) * 8 * sd::kHeadDim * 2;
    if (h[0] > 0) {
        const int par = int((h[0] - 1) & 1);
        out->last_needed = h[4 + 4 * par];
        out->last_hits = h[5 + 4 * par];
        out->last_misses = h[6 + 4 * par];
        out->last_refills = h[7 + 4 * par];
    }
    out->last_copies = c->vfetch == SD_VALUE_FETCH_COPY ? c->vcopies : 0;
    return SD_OK;
}

sd_status sd_reset_value_cache(sd_ctx* c, void* stream) {
    if (!c) return SD_ERR_INVALID_ARG;
    if (!c->cfg.values_on_host) return SD_OK;
    return from_hip(sd::launch_value_cache_reset(c, static_cast<hipStream_t>(stream)));
}

sd_status sd_profile_start(sd_ctx* c, uint32_t kind_mask, int32_t max_launches) {
    if (!c || max_launches < 1 || max_launches > (1 << 20)) return SD_ERR_INVALID_ARG;
    free_profiler(c);
    c->prof_ev = new (std::nothrow) hipEvent_t[2 * size_t(max_launches)]();
    c->prof_kind = new (std::nothrow) int8_t[size_t(max_launches)]();
    if (!c->prof_ev || !c->prof_kind) { free_profiler(c); return SD_ERR_OUT_OF_MEMORY; }
    c->prof_max = max_launches;
    for (int i = 0; i < 2 * max_launches; ++i) {
        if (hipEventCreate(&c->prof_ev[i]) != hipSuccess) { free_profiler(c); return SD_ERR_HIP; }
    }
    c->prof_mask = kind_mask;
    c->prof_n = 0;
    return SD_OK;
}

sd_status sd_profile_stop(sd_ctx* c, sd_profile* out) {
    if (!c) return SD_ERR_INVALID_ARG;
    sd_profile r;
    std::memset(&r, 0, sizeof(r));
    hipError_t e = c->prof_ev ? hipDeviceSynchronize() : hipSuccess;
    for (int i = 0; e == hipSuccess && i < c->prof_n; ++i) {
        float ms = 0.f;
        e = hipEventElapsedTime(&ms, c->prof_ev[2 * i], c->prof_ev[2 * i + 1]);
        r.ms[c->prof_kind[i]] += ms;
        r.launches[c->prof_kind[i]] += 1;
    }
    free_profiler(c);
    if (out) *out = r;
    return from_hip(e);
}

}  // extern "C"
