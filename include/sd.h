/*
 * sd.h -- C ABI of the sparse decode-attention library (libsd.so).
 *
 * One decode step of attention over a long KV cache, in three parts:
 *
 *  1. Keys are quantised once to symmetric int8 with one absmax scale per
 *     (request, KV head).  Sources: summary page of "HCAttention: Extreme KV
 *     cache compression via heterogeneous attention computing for LLMs",
 *     sections 摘要 and 引言 (quantised keys stay on the GPU and drive a
 *     global approximate scoring); page "KV Cache 与长上下文推理", section
 *     "KV Cache 压缩技术" (INT8 key cache).
 *  2. Stacked pruning stages rank fixed-length chunks by one representative
 *     score each and keep the top K chunks, refining chunk length stage by
 *     stage.  Source: news article on InfiniteHiP ("韩国通过卸载键值缓存节约
 *     英伟达GPU内存，实现18.95倍解码加速"), section "实现 7.24 倍的端到端解码加速".
 *     A chunk's score is the maximum, over tokens sampled at the stage's
 *     stride from the chunk start, of the exact integer dot product between
 *     the int8 key and the sum of the group's int8 query vectors; ties go
 *     to the lower chunk start.
 *  3. Exact GQA attention (bf16 q and K, fp32 accumulation, bf16 output)
 *     over the kept chunks plus the first `sink` and last `window` tokens.
 *     Sources: page "KV Cache 与长上下文推理", section "KV Cache 回顾" (decode
 *     attention equation) and section "KV Cache 压缩技术" (GQA table;
 *     StreamingLLM sink + sliding window).
 *
 * Optionally values live in pinned host memory behind an LRU cache of
 * 8-token value blocks in device memory (news article on InfiniteHiP, same
 * section: LRU-based offload; HCAttention summary, section 引言: values in
 * CPU memory, fetched late for the final aggregation).
 *
 * Conventions for every call:
 *  - bf16 tensors are passed as uint16_t bit patterns.
 *  - "device" pointers are device memory of the context's GPU; "host"
 *    pointers are ordinary host memory.  The caller owns every buffer it
 *    passes; the context owns its workspace (allocated in sd_create only).
 *  - Work is enqueued on the caller's HIP stream (`stream`, a hipStream_t;
 *    NULL = the null stream) and the call returns without waiting, except
 *    where a call says it synchronises.
 *  - Calls return a status and never abort.  Argument and configuration
 *    errors are reported synchronously.  Bad values found on the device
 *    (a length outside [1, max_context]) set a flag reported by sd_check.
 *  - A context is used from one host thread and one stream at a time.
 */
#ifndef SD_H_
#define SD_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct sd_ctx sd_ctx;

typedef enum sd_status {
    SD_OK = 0,
    SD_ERR_INVALID_ARG = 1,     /* null pointer, bad size or inconsistent config */
    SD_ERR_UNSUPPORTED = 2,     /* valid but outside what the kernels implement */
    SD_ERR_OUT_OF_MEMORY = 3,   /* workspace allocation failed in sd_create */
    SD_ERR_HIP = 4,             /* a HIP runtime call failed */
    SD_ERR_DEVICE_FLAG = 5      /* a kernel flagged bad input (see sd_check) */
} sd_status;

#define SD_MAX_STAGES 4

/* One pruning stage: chunks of `chunk` tokens, representative sampled every
 * `stride` tokens from the chunk start, the `keep` best chunks survive.
 * Stage 1 chunks start at 0, chunk, 2*chunk, ...; the chunks of stage s+1
 * are the sub-chunks of the survivors of stage s. */
typedef struct sd_stage {
    int32_t chunk;
    int32_t stride;
    int32_t keep;
} sd_stage;

typedef struct sd_config {
    int32_t batch;              /* B >= 1 */
    int32_t num_q_heads;        /* Hq */
    int32_t num_kv_heads;       /* Hkv; Hq = G * Hkv with G in {1, 2, 4} */
    int32_t head_dim;           /* d; must be 128 */
    int64_t max_context;        /* Lmax: token stride of every [B][Hkv][Lmax][d] buffer */
    int32_t num_stages;         /* S in [1, SD_MAX_STAGES] */
    sd_stage stage[SD_MAX_STAGES];
    /* Requirements: stride divides chunk; chunk[s+1] divides chunk[s];
     * the last stage's chunk is a multiple of 8; keep >= 1;
     * chunk / stride <= 64 at every stage; for every stage the number of
     * candidates n_s (n_0 = ceil(Lmax / chunk[0]), n_s = keep[s-1] *
     * chunk[s-1] / chunk[s]) plus keep[s] is at most 15872. */
    int32_t sink;               /* first `sink` tokens always attended (>= 0) */
    int32_t window;             /* last `window` tokens always attended (>= 0) */
    float softmax_scale;        /* 0 selects 1 / sqrt(head_dim) */
    int32_t values_on_host;     /* 0: v is device memory; 1: v is pinned host memory */
    int64_t value_cache_tokens; /* values_on_host: device cache size in tokens per
                                   (request, KV head); a multiple of 8 that holds at
                                   least one step's attended blocks */
} sd_config;

/* Counters of the host-value path (values_on_host = 1), over all steps
 * since creation or the last sd_reset_value_cache, and for the last step.
 * A refill is a hit whose cached block was written when fewer of its rows
 * were below the length than now (the length grew since): the block is
 * read from host memory again.  It counts as a hit of the LRU policy. */
typedef struct sd_stats {
    int64_t steps;
    int64_t blocks_needed;      /* sum over steps and (request, KV head) of |blocks of T| */
    int64_t hits;
    int64_t misses;
    int64_t h2d_bytes;          /* (misses + refills) * 8 tokens * d * 2 bytes read from host memory */
    int64_t last_needed;
    int64_t last_hits;
    int64_t last_misses;
    int64_t refills;
    int64_t last_refills;
    int64_t last_copies;        /* SD_VALUE_FETCH_COPY: hipMemcpyAsync calls of the last step (else 0) */
} sd_stats;

/* Creates a context on the current HIP device, validating `cfg` and
 * allocating all device workspace (no later call allocates).  On success
 * *out receives the context; on failure *out is set to NULL.
 * The context's launch plan (which changes no result) is fixed here and
 * read from these environment variables, when set:
 *  SD_FUSE_LAST_STAGE=0 / =1  never / always (where the stage geometry
 *                             allows) score the last stage inside the
 *                             kernel of the stage before it; default: when
 *                             the extra key rows stay within 8 MiB.
 *  SD_HALF_ROWS=0             unfused, with the stage before the last
 *                             sampling every other row of the last stage's
 *                             8-row chunks: the last stage reads all eight
 *                             rows; default with 32 or more (request, KV
 *                             head) pipelines: only the four that stage did
 *                             not read, the other four's maximum stored by it.
 *  SD_VCACHE_ONCHIP=0         host values: the LRU step through device
 *                             memory at every cache size; default: on chip
 *                             for at most 8,192 slots and 1,024 attended
 *                             blocks per (request, KV head).
 *  SD_DENSE_WG_PER_CU=n       sd_dense_decode's workgroups per CU
 *                             (default 8). */
sd_status sd_create(const sd_config* cfg, sd_ctx** out);

/* Releases the context and its workspace after the device is idle.
 * NULL is a no-op. */
void sd_destroy(sd_ctx* ctx);

/* Static text for a status code. */
const char* sd_status_string(sd_status status);

/* Text of the last HIP failure seen by this thread ("" if none): the HIP
 * call and its error string.  Valid until the thread's next library call. */
const char* sd_last_error(void);

/* Quantises the key cache (part 1).
 *  k_bf16   device [B][Hkv][Lmax][d] bf16 keys.
 *  lengths  device [B] int32 request lengths L_b in [1, Lmax].
 *  k_int8   device [B][Hkv][Lmax][d] int8 output: for t < L_b the code
 *           rint(127 * k / a_bj) (round half to even, correctly rounded
 *           fp32 division), a_bj = max |k| over t < L_b and all channels
 *           (codes are 0 when a_bj = 0).  Rows t >= L_b are not written.
 *  k_absmax device [B][Hkv] fp32 output a_bj, or NULL. */
sd_status sd_quantize_keys(sd_ctx* ctx, const uint16_t* k_bf16, const int32_t* lengths,
                           int8_t* k_int8, float* k_absmax, void* stream);

/* Appends n_new tokens per request to the caches, as a decode loop does
 * after each step (the pages keep the cache growing by one token per decode
 * step: page "KV Cache 与长上下文推理", section "KV Cache 回顾"; they say
 * nothing of how a quantised cache's scale follows that growth).  The key
 * scale is a running absmax: the new keys of (request b, KV head j) are
 * coded with a' = max(a_bj, absmax of the new keys), and when a' > a_bj
 * every earlier row of that (b, j) is recoded with a' on the device.  So
 * after the call the codes and scales equal what sd_quantize_keys gives for
 * the grown cache (t < L_b + n_new), bit for bit.  a_bj is the scale this
 * context holds for the cache: the one sd_quantize_keys (or an earlier
 * sd_append_kv) on this context computed; the call continues that cache.
 *  k_new    device [B][Hkv][n_new][d] bf16 new keys.
 *  v_new    device [B][Hkv][n_new][d] bf16 new values.
 *  n_new    tokens per request, in [1, Lmax].
 *  lengths  device [B] int32: the lengths L_b BEFORE the append (not
 *           modified: the caller passes L_b + n_new to the next call).
 *  k_bf16, k_int8, v  device caches ([B][Hkv][Lmax][d]); rows
 *           [L_b, L_b + n_new) are written (all rows t < L_b + n_new of
 *           k_int8 when the scale grew).
 *  k_sketch4 device int4 first-stage sketch (see sd_quantize_sketch4) kept
 *           up to date as well, or NULL: the new rows t that are multiples
 *           of stage[0].stride are coded into it, and when a scale grew all
 *           of that (request, KV head)'s sketch rows are recoded, so it
 *           equals sd_quantize_sketch4 of the grown cache.
 *  k_absmax device [B][Hkv] fp32 output a', or NULL.
 * A request with L_b < 1 or L_b + n_new > Lmax is left untouched and
 * raises the device flag (see sd_check).  Needs values_on_host = 0 (else
 * SD_ERR_UNSUPPORTED).  Allocates nothing. */
sd_status sd_append_kv(sd_ctx* ctx, const uint16_t* k_new, const uint16_t* v_new, int32_t n_new,
                       const int32_t* lengths, uint16_t* k_bf16, int8_t* k_int8, uint16_t* v,
                       uint8_t* k_sketch4, float* k_absmax, void* stream);

/* One decode step (parts 2 and 3).
 *  q        device [B][Hq][d] bf16 query of the step.
 *  k_bf16   device [B][Hkv][Lmax][d] bf16 keys (exact attention).
 *  k_int8   device [B][Hkv][Lmax][d] int8 keys from sd_quantize_keys.
 *  v        [B][Hkv][Lmax][d] bf16 values: device memory, or pinned host
 *           memory (allocated with hipHostMalloc) when values_on_host = 1.
 *  lengths  device [B] int32, each in [1, Lmax].
 *  out      device [B][Hq][d] bf16 attention output.
 *  kept_idx device [B][Hkv][sum_s keep_s] int32: stage s occupies offset
 *           sum_{u<s} keep_u and holds its kept chunk starts (token
 *           positions) ascending, padded with -1.
 * Query head h uses KV head h / G.  A request with a length outside
 * [1, Lmax] gets zero output and -1 indices, and raises the device flag. */
sd_status sd_decode_step(sd_ctx* ctx, const uint16_t* q, const uint16_t* k_bf16,
                         const int8_t* k_int8, const uint16_t* v, const int32_t* lengths,
                         uint16_t* out, int32_t* kept_idx, void* stream);

/* sd_decode_step for callers that cannot allocate device memory: code being
 * captured into a HIP graph, tight serving loops, harnesses that forbid
 * hipMalloc.  It takes the configuration instead of a context and allocates
 * nothing (no hipMalloc, hipFree or allocating library call): the step's
 * workspace (chunk scores, group query sums, split partials and the error
 * flag) lives in a fixed 16 MiB array of device memory that the library
 * holds on every GPU it runs on until the process ends; its address on each
 * GPU is looked up on the first call there.  Arguments and results are
 * those of sd_decode_step on a context created from *cfg (same kernels,
 * bit-identical outputs and kept_idx).
 *  cfg      host pointer, read during the call only; values_on_host must be
 *           0 (SD_ERR_UNSUPPORTED otherwise: the value cache needs a
 *           context).  A configuration whose workspace exceeds the 16 MiB
 *           (many requests at long contexts) gets SD_ERR_UNSUPPORTED with
 *           the sizes in sd_last_error(); about 1.3 MiB serve one request at
 *           1M tokens (GQA 32/8), about 3 MiB sixteen requests of 128K.
 * Every call on a GPU uses that GPU's one array: calls that overlap on one
 * GPU (other streams, other threads) race and give wrong results; calls in
 * one stream order are safe.  The error flag is cleared by the call itself;
 * a length outside [1, Lmax] gives zero output and -1 indices, as in
 * sd_decode_step, but no sd_check can report it (there is no context). */
sd_status sd_decode_step_noalloc(const sd_config* cfg, const uint16_t* q, const uint16_t* k_bf16,
                                 const int8_t* k_int8, const uint16_t* v, const int32_t* lengths,
                                 uint16_t* out, int32_t* kept_idx, void* stream);

/* sd_decode_step with the first `reuse_stages` pruning stages reused from an
 * earlier step: news article on InfiniteHiP ("韩国通过卸载键值缓存节约英伟达GPU
 * 内存，实现18.95倍解码加速"), section "实现 7.24 倍的端到端解码加速": the modular
 * design allows fine-grained control over caching the pruning stages, for
 * faster decoding.  Stages s < reuse_stages are not run: their kept sets are
 * the ones kept_idx holds (as an earlier step on the same kept_idx left
 * them), and stage reuse_stages takes its candidates from the children of
 * stage reuse_stages - 1's kept chunks that start before the current
 * length.  Later stages, the attended set and the attention run as in
 * sd_decode_step, with this step's query.  reuse_stages = 0 is
 * sd_decode_step; reuse_stages = num_stages reuses every stage and runs
 * only the attention.
 *  reuse_stages  in [0, num_stages], else SD_ERR_INVALID_ARG.
 * kept_idx is read as well as written: the entries of reused stages are
 * left as they are; entries outside [0, length) are ignored.  kept sets not
 * written by a step of this context (unsorted, repeated, or not multiples
 * of the chunk) give unspecified results but no out-of-range access.
 * Chunk scores of reused stages (sd_stage_scores) stay those of the step
 * that computed them. */
sd_status sd_decode_step_reuse(sd_ctx* ctx, const uint16_t* q, const uint16_t* k_bf16,
                               const int8_t* k_int8, const uint16_t* v, const int32_t* lengths,
                               uint16_t* out, int32_t* kept_idx, int32_t reuse_stages,
                               void* stream);

/* Dense decode attention over every cached token, for comparison with the
 * sparse step: for each query head h, softmax(softmax_scale * q_h K^T) V
 * over all tokens t < L_b of KV head h / G, with the same arithmetic as the
 * sparse step's attention (bf16 q and K, fp32 scores, online softmax and
 * accumulation, log-sum-exp merge of the splits, bf16 output rounded to
 * nearest even).  Sources: page "KV Cache 与长上下文推理", section "KV Cache
 * 回顾" (the decode attention equation over the whole cache); the news
 * article on InfiniteHiP, opening section, compares its sparse decoding
 * against exactly this dense attention at long context.
 *  q        device [B][Hq][d] bf16.
 *  k_bf16   device [B][Hkv][Lmax][d] bf16 keys.
 *  v        device [B][Hkv][Lmax][d] bf16 values.
 *  lengths  device [B] int32, each in [1, Lmax].
 *  out      device [B][Hq][d] bf16 output.
 * Needs values_on_host = 0 (else SD_ERR_UNSUPPORTED).  Uses the context's
 * workspace for its split partials, so it must not overlap a decode step of
 * the same context.  A request with a length outside [1, Lmax] gets zero
 * output and raises the device flag (see sd_check).  Allocates nothing. */
sd_status sd_dense_decode(sd_ctx* ctx, const uint16_t* q, const uint16_t* k_bf16,
                          const uint16_t* v, const int32_t* lengths, uint16_t* out,
                          void* stream);

/* int4 scoring keys for the first pruning stage (the notes page "KV Cache 与
 * 长上下文推理", section "KV Cache 压缩技术", lists INT4 next to INT8 as a
 * cache quantisation; here it is applied to the first stage's scoring
 * only, the stage that reads the most key rows).  The sketch holds the rows
 * the first stage samples, t = i * r_1 (r_1 = stage[0].stride), i <
 * ceil(L_b / r_1): codes c = rint(7 * k / a_bj) in [-7, 7] (round half to
 * even, correctly rounded fp32 division) with the key scale a_bj of
 * sd_quantize_keys, stored as two's-complement nibbles; byte m of a row
 * holds channel 2m in its low and channel 2m + 1 in its high nibble (64
 * bytes per row).
 *
 * Rows per (request, KV head) of the sketch: ceil(Lmax / r_1). */
int64_t sd_sketch4_rows(const sd_ctx* ctx);

/* Writes the sketch of the cache whose scales the context holds (the last
 * sd_quantize_keys on this context, and the sd_append_kv calls after it;
 * an append given the sketch keeps it up to date).
 *  k_bf16     device [B][Hkv][Lmax][d] bf16 keys.
 *  lengths    device [B] int32 in [1, Lmax] (other requests are skipped).
 *  k_sketch4  device [B][Hkv][sd_sketch4_rows][64] uint8 output; rows
 *             i >= ceil(L_b / r_1) are not written. */
sd_status sd_quantize_sketch4(sd_ctx* ctx, const uint16_t* k_bf16, const int32_t* lengths,
                              uint8_t* k_sketch4, void* stream);

/* sd_decode_step with the first stage scored from the sketch: its chunk
 * score is the max over its samples t of S4_t = Q_j . K4_(t / r_1) (exact
 * integer; Q_j as in sd_decode_step); every later stage, the attended set
 * and the attention are those of sd_decode_step.  Arguments as in
 * sd_decode_step, plus k_sketch4 from sd_quantize_sketch4.  Needs the first
 * stage to run unfused: SD_ERR_UNSUPPORTED for a 2-stage configuration
 * whose last stage the context fuses into the first (sd_create fuses the
 * last stage into the one before it, where the geometry allows, when the
 * extra key rows that costs over all (request, KV head) pairs stay within
 * 8 MiB; the environment variable SD_FUSE_LAST_STAGE=0 turns fusion off,
 * =1 fuses wherever the geometry allows). */
sd_status sd_decode_step_sketch4(sd_ctx* ctx, const uint16_t* q, const uint16_t* k_bf16,
                                 const int8_t* k_int8, const uint8_t* k_sketch4, const uint16_t* v,
                                 const int32_t* lengths, uint16_t* out, int32_t* kept_idx,
                                 void* stream);

/* The step's query codes, for inspection: q8 device [B][Hq][d] int8 with one
 * absmax scale per query head (same rounding as the keys), and q_group
 * device [B][Hkv][d] int32, the sum of q8 over each KV head's group.  Either
 * output may be NULL.  Uses the same device code as sd_decode_step. */
sd_status sd_quantize_query(sd_ctx* ctx, const uint16_t* q, int8_t* q8, int32_t* q_group,
                            void* stream);

/* Records the attended set as the decode kernel walks it, for inspection:
 * from the next sd_decode_step / sd_decode_step_reuse / sd_decode_step_sketch4
 * of this context on, until called with dst = NULL, each 8-token block the
 * kernel's block loop attends is stored as one word, block << 8 | mask
 * (block = first token / 8; bit i of the 8-bit mask set when token
 * 8 block + i is attended), into device memory dst laid out
 * [B][Hkv][max_blocks], max_blocks = keep_last * chunk_last / 8 +
 * ceil(sink / 8) + ceil(window / 8) + 1.  Device values: words
 * [0, keep_last * chunk_last / 8) of a (request, KV head) are the blocks of
 * the last stage's kept chunks (in kept order, sink and window tokens
 * masked out), words from keep_last * chunk_last / 8 on are the sink and
 * window blocks; host values: the attended block list.  So the union of the
 * masks is the attended set (kept last-stage chunks, sink and window:
 * "KV Cache 与长上下文推理", section "KV Cache 压缩技术"), each token once.
 * Words the step does not write keep their value: clear dst before a step.
 * The caller keeps dst alive while recording is on; the words are stored by
 * the same block loop that loads the keys and values.
 *  SD_ERR_INVALID_ARG  dst_len < B * Hkv * max_blocks.
 *  SD_ERR_UNSUPPORTED  max_context > 2^27 (block ids must fit 24 bits). */
sd_status sd_record_attended(sd_ctx* ctx, uint32_t* dst, int64_t dst_len);

/* Copies the chunk scores stage `stage` (0-based) computed by the last
 * sd_decode_step into device memory `dst`, laid out [B][Hkv][n_stage] int32
 * (n_0 = ceil(Lmax / chunk_0), n_s = keep_{s-1} * chunk_{s-1} / chunk_s);
 * entries of chunks that do not exist hold INT32_MIN.  For inspection. */
sd_status sd_stage_scores(sd_ctx* ctx, int32_t stage, int32_t* dst, int64_t dst_len,
                          void* stream);

/* Number of int32 entries per (request, KV head) of sd_stage_scores. */
int64_t sd_stage_candidates(const sd_ctx* ctx, int32_t stage);

/* Synchronises `stream`, then reports SD_ERR_DEVICE_FLAG (and clears the
 * flag) if a kernel flagged bad input since the last check, else SD_OK. */
sd_status sd_check(sd_ctx* ctx, void* stream);

/* Synchronises `stream` and fills *stats (host-value path counters; all
 * zero when values_on_host = 0). */
sd_status sd_get_stats(sd_ctx* ctx, sd_stats* stats, void* stream);

/* Empties the value cache and zeroes the counters (enqueued on `stream`). */
sd_status sd_reset_value_cache(sd_ctx* ctx, void* stream);

/* How missed value blocks reach the device (values_on_host = 1).
 *  SD_VALUE_FETCH_MAPPED (default): the decode kernel reads each missed
 *    block from pinned host memory through its device alias and writes it
 *    into the block's slot, in the same pass that attends it; the step
 *    stays asynchronous and graph-capturable.
 *  SD_VALUE_FETCH_COPY: the gathered-copy design (HCAttention, section 引言:
 *    values kept in CPU memory and fetched late, for the final weighted
 *    sum; news article on InfiniteHiP, section "解决长上下文推理问题，能通过键值
 *    缓存卸载节约 GPU 内存": offloaded KV blocks fetched on demand): after
 *    the value-cache kernel, the host waits for the step's block list,
 *    enqueues one hipMemcpyAsync per run of missed blocks (consecutive in
 *    host memory and in the slot pool) on a side stream of the context,
 *    and the decode kernel, ordered after those copies by an event, reads
 *    every block from the slot pool.  Same LRU, same results; the step
 *    synchronises the host once and cannot be captured in a graph
 *    (SD_ERR_UNSUPPORTED while `stream` is capturing).
 * SD_ERR_UNSUPPORTED if values_on_host = 0; SD_ERR_INVALID_ARG for another
 * mode.  Takes effect from the next step. */
#define SD_VALUE_FETCH_MAPPED 0
#define SD_VALUE_FETCH_COPY 1
sd_status sd_set_value_fetch(sd_ctx* ctx, int32_t mode);

/* Kernel kinds timed by the profiler. */
enum {
    SD_PROF_STAGE0 = 0,         /* pruning stage s is SD_PROF_STAGE0 + s */
    SD_PROF_VALUE_CACHE = 4,    /* LRU update of the host-value path */
    SD_PROF_ATTEND = 5,         /* last select + attended set + sparse flash decode + merge of its splits */
    SD_PROF_QUANTIZE = 6,       /* the three kernels of sd_quantize_keys, as one interval */
    SD_PROF_COMBINE = 7,        /* log-sum-exp merge of the dense decode's splits into the bf16 output */
    SD_PROF_DENSE = 8,          /* dense flash decode of sd_dense_decode (partials; its merge is COMBINE) */
    SD_PROF_APPEND = 9,         /* the two kernels of sd_append_kv, as one interval */
    SD_PROF_KINDS = 10
};

typedef struct sd_profile {
    float ms[SD_PROF_KINDS];        /* summed device time between the bracketing events */
    int32_t launches[SD_PROF_KINDS];
} sd_profile;

/* Starts timing: while active, every launch of a kind whose bit is set in
 * `kind_mask` carries a start and a stop HIP event in its own dispatch on
 * the caller's stream (no separate marker packets), for at most
 * `max_launches` launches.  Allocates the events (host call; not to be used
 * where allocation is forbidden). */
sd_status sd_profile_start(sd_ctx* ctx, uint32_t kind_mask, int32_t max_launches);

/* Stops timing: synchronises the device, sums the elapsed times per kind
 * into *out (may be NULL) and frees the events. */
sd_status sd_profile_stop(sd_ctx* ctx, sd_profile* out);

#ifdef __cplusplus
}
#endif

#endif /* SD_H_ */
