/*
 * routed_moe.h -- C ABI of the routed Mixture-of-Experts layer executed over a
 * bounded GPU expert cache shared by every MoE layer (AMD MI355X, gfx950).
 *
 * Per MoE layer the method runs: router softmax/top-k; a lookup from the
 * logical (layer, expert) id to a cache slot with LRU update; token permutation
 * by expert; the SwiGLU expert FFN on resident slots; a gate-weighted combine.
 * Misses are either filled over PCIe from a pinned host expert pool or run on
 * host CPU cores, split by q* = m * B_P / B_H.
 *
 * Sources, cited by page title and section:
 *   [FT-KR] FreeToken paper summary, discuss.pytorch.kr ("FreeToken: ...
 *           Edge-Serving에 대한 연구").
 *   [FT-CN] FreeToken reading notes, qqtang-code.github.io ("论文精读 ·
 *           FreeToken: 边缘原生的 MoE 服务系统").
 *   [SPARK] "Luce Spark" expert-offload post, molayo1419.me.
 *
 * Conventions for every call:
 *  - Every call returns moe_status (0 = MOE_OK, negative = error) unless noted.
 *    No C++ exception crosses this boundary.  moe_last_error() gives the text
 *    of the last error on a context.
 *  - "device" pointers are HIP device allocations on the context's device; "host"
 *    pointers are CPU memory.  The caller owns every pointer it passes in (inputs,
 *    outputs, router weights, slot arena, a registered host pool) and must keep it
 *    alive while the context may use it.  The library owns the residency tables,
 *    work lists, pinned staging, a copy stream, events and the CPU worker pool.
 *  - Calls on one context must be serialised by the caller.  Work is enqueued on
 *    the stream argument (a hipStream_t; NULL = the null stream).  Calls that need
 *    a host decision (fills, CPU branch, resize) synchronise on that stream.
 *  - Device-side faults surface as MOE_EHIP at the next synchronising call.
 *  - Tokens are rows: x is [T, hidden] row-major in the activation format; y is
 *    [T, hidden] fp32.  topk_idx / topk_w / slot_idx are [T, top_k] row-major.
 */
#ifndef ROUTED_MOE_H
#define ROUTED_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_API __attribute__((visibility("default")))

typedef struct moe_ctx moe_ctx;
typedef void* moe_stream_t; /* hipStream_t */

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = -1,  /* bad argument, shape or size */
  MOE_ENOMEM = -2,  /* allocation failed */
  MOE_EHIP = -3,    /* HIP runtime error (includes device faults) */
  MOE_ESTATE = -4,  /* call-order violation (e.g. decode without lookup, resize in prefill) */
  MOE_ENOPIN = -5,  /* the host pool is not page-locked: only MOE_MODE_CPU can use it */
  MOE_ENOTSUP = -6, /* combination not supported */
  MOE_ETIMEDOUT = -7 /* a captured step's bounded wait for its CPU branch expired (moe_sync) */
} moe_status;

/* Expert weight formats of a pool record (see moe_record_bytes for the layout). */
typedef enum {
  MOE_WFMT_F32 = 0,  /* fp32 gate | up | down */
  MOE_WFMT_BF16 = 1, /* bf16 gate | up | down */
  MOE_WFMT_FP4 = 2,  /* e2m1 codes + one bf16 scale per 32 elements along each row */
  MOE_WFMT_MXFP4 = 3 /* e2m1 codes + one E8M0 scale byte per 32 elements (the MX format of the
                        pages' DeepSeek-V4-Flash experts, [FT-KR] "실험 환경"); hidden and inter
                        must be multiples of 256 */
} moe_wfmt;

typedef enum { MOE_AFMT_F32 = 0, MOE_AFMT_BF16 = 1 } moe_afmt;

/*
 * Arithmetic and the intermediates rounded to 16 bits (every rounding is to nearest even;
 * accumulation is fp32 everywhere):
 *  decode gate/up: bf16 activations with bf16 / FP4 / MXFP4 weights multiply exactly
 *    (v_dot2_f32_bf16; e2m1 codes become bf16 exactly, a bf16 block scale multiplies the fp32
 *    block sum, an E8M0 scale is applied exactly by the convert); other combinations in fp32.
 *  decode down projection: with bf16 / FP4 / MXFP4 weights, the SwiGLU intermediate h is
 *    rounded to bf16 when a row of W_down is one 16-byte load per lane (inter = 2048 for e2m1
 *    rows, 512 for bf16), T <= 4 and T*k <= 64; otherwise, and with fp32 weights, h stays fp32.
 *  prefill, FP4 / MXFP4 weights: activations become f16, each weight (code x block scale)
 *    is formed in f16, h is stored as f16 between the two GEMMs (f16 MFMA, fp32 accumulate).
 *    These are exact only while the values lie in f16's normal range (magnitudes in
 *    [2^-14, 65504]): larger ones overflow and smaller ones lose bits, with no error
 *    reported, so FP4 pools with block scales, or activations, outside that range need the
 *    bf16 format.  bf16 weights: bf16 activations and weights, h stored as bf16.  fp32
 *    weights: fp32 throughout.
 *  CPU branch: fp32 throughout (h is not rounded), so a HYBRID step's CPU and GPU experts
 *    can differ in the last bits of h's rounding.
 */

/*
 * Backend modes ([FT-KR] usage section: --moe-backend fused|offload|cpu|hybrid):
 *  FUSED   every record is resident; slot = key; no cache.
 *  OFFLOAD LRU cache; every miss is filled over PCIe (capped by evictable slots).
 *  CPU     LRU cache for hits; every miss runs on the host CPU.
 *  HYBRID  misses split by q* between fills and the CPU.
 */
typedef enum { MOE_MODE_FUSED = 0, MOE_MODE_OFFLOAD = 1, MOE_MODE_CPU = 2, MOE_MODE_HYBRID = 3 } moe_mode;

/* Trace record kinds: hit, fill, CPU execution, prefill full-layer buffer. */
typedef enum { MOE_KIND_HIT = 0, MOE_KIND_FILL = 1, MOE_KIND_CPU = 2, MOE_KIND_BUF = 3 } moe_kind;

#define MOE_FLAG_PROFILE 1 /* time the FFN kernels with HIP events (moe_get_stats) */
/* Cached decode steps copy their fills with a kernel that reads the page-locked pool through
 * its device mapping; captured steps hand their CPU branch to a library thread, so replay
 * has no host node (see moe_ffn_decode). */
#define MOE_FLAG_DEVICE_FILLS 2
/* MXFP4 experts only (else moe_create returns MOE_ENOTSUP): the prefill GEMMs on the GPU take
 * their activation operands in MXFP8 and multiply them with the weights' e2m1 codes and E8M0
 * scales as stored (gfx950 v_mfma_scale_f32_32x32x64_f8f6f4, fp32 accumulation).  The pages
 * leave the activation format open ([FT-KR] "실험 환경" serves the experts in MXFP4); the
 * conversion is that of the OCP Microscaling v1.0 specification: 32-element blocks along the
 * reduction dimension, E8M0 scale 2^(floor(log2 max|v|) - 8) (clamped to [-127, 127]; -127 for
 * a block of zeros), E4M3 elements rounded to nearest even and saturated at 448; the SwiGLU
 * intermediate is converted from its fp32 value.  Decode and experts a CPU or HYBRID prefill
 * round sends to the host keep their own arithmetic. */
#define MOE_FLAG_MX_PREFILL 4

typedef struct {
  int32_t n_layers, n_experts, top_k, hidden, inter; /* L, E, k, H, I */
  int32_t wfmt;        /* moe_wfmt */
  int32_t afmt;        /* moe_afmt */
  int32_t renorm;      /* 0: gates are the softmax over all E; 1: renormalised over the k chosen */
  int32_t max_tokens;  /* largest T any call will pass */
  int32_t mode;        /* moe_mode */
  uint64_t bw_pcie;    /* B_P, bytes/s (host -> device expert transfer) */
  uint64_t bw_host;    /* B_H, bytes/s (host CPU expert processing) */
  int32_t cpu_threads; /* CPU branch threads; 0 = the CPUs of the process affinity mask but two */
  int32_t flags;       /* MOE_FLAG_* */
} moe_config;

/* One record per distinct routed key of a layer step, in first-appearance order
 * over (token, rank) pairs.  slot = -1 for CPU; evicted = key that lost the slot, or -1. */
typedef struct {
  int32_t key, kind, slot, evicted;
} moe_trace_rec;

/* Counters returned by lookups (all int32). */
enum { MOE_CNT_HIT = 0, MOE_CNT_FILL = 1, MOE_CNT_CPU = 2, MOE_CNT_EVICT = 3 };

typedef struct {
  uint64_t decode_calls, prefill_calls, lookups;
  uint64_t hits, fills, cpu_experts, evictions;
  uint64_t fill_bytes;            /* bytes copied host -> slot arena */
  double phase1_ms, phase2_ms;    /* summed kernel time (MOE_FLAG_PROFILE) */
  uint64_t phase1_launches, phase2_launches;
  uint64_t phase1_bytes, phase2_bytes; /* algorithmic weight + activation bytes of those launches */
  double gemm1_ms, gemm2_ms;      /* prefill grouped GEMMs (MOE_FLAG_PROFILE) */
  uint64_t gemm1_launches, gemm2_launches;
  double gemm_flops;              /* algorithmic flops of those launches: 2 * pairs * 3 * H * I */
  double copy_ms;                 /* prefill whole-layer copies (MOE_FLAG_PROFILE) */
  uint64_t copy_bytes;
  double cpu_ms;                  /* host CPU branch wall time */
} moe_stats;

/* ---- context ---------------------------------------------------------- */

/* Create a context on the current HIP device.  Validates the shape: top_k <= n_experts <= 1024,
 * hidden % 64 == 0 and inter % 64 == 0 (FP4 also needs multiples of 32 along rows), max_tokens >= 1. */
MOE_API moe_status moe_create(const moe_config* cfg, moe_ctx** out);
MOE_API moe_status moe_destroy(moe_ctx* ctx);
/* Text of the last error on ctx (never NULL; "" when none).  Valid until the next call on ctx. */
MOE_API const char* moe_last_error(const moe_ctx* ctx);

/*
 * Bytes S of one expert record, the unit of every fill and of the host pool.
 * A slot holds every tensor of one (layer, expert) pair ([FT-KR] "FreeToken의 설계"),
 * so one record moves one expert.  Layout (row-major, W_gate/W_up [I,H], W_down [H,I]):
 *   F32 / BF16: [gate | up | down], element size 4 / 2
 *   FP4:        [gate codes I*H/2 | up codes | down codes H*I/2 | gate scales I*H/32 bf16 |
 *                up scales | down scales]; element 2i of a row is the low nibble of byte i;
 *                one scale per 32 consecutive elements of a row (the reduction dimension);
 *                w = e2m1(code) * scale.
 *   MXFP4:      as FP4 with one scale byte e per block (E8M0, bias 127): w = e2m1(code) * 2^(e-127);
 *                e must lie in 1..254.
 * Returns -1 for an invalid config.  Pure host function.
 */
MOE_API int64_t moe_record_bytes(const moe_config* cfg);

/*
 * Whether n_records records at `pool` (host memory laid out as moe_record_bytes defines,
 * caller-owned, only read) keep the FP4 / MXFP4 prefill exact.  The prefill forms every
 * weight e2m1(code) x scale in f16 (see the arithmetic note above), which is exact while
 * each nonzero weight lies in f16's normal range [2^-14, 65504].  Only the block scales are
 * read, and any code is assumed to occur in a block, so a nonzero scale s must satisfy
 * 0.5 |s| >= 2^-14 and 6 |s| <= 65504: bf16 scales in [2^-13, 10880] (or zero), E8M0 bytes
 * in 114..140.  Records outside that range still decode exactly (fp32 arithmetic); their
 * prefill weights overflow or lose bits with no error, so such pools need the bf16 format.
 * *first_bad receives the lowest failing record index, or -1.  MOE_OK when every record
 * passes (always for fp32 and bf16 weights), MOE_EINVAL when one fails or for a bad
 * argument.  Pure host function (several threads for a large pool).
 */
MOE_API moe_status moe_pool_check_f16(const moe_config* cfg, const void* pool, int64_t n_records,
                                      int64_t* first_bad);

/* ---- host expert pool (the source of truth) ---------------------------- */

/*
 * Allocate a page-locked host pool of n_records records owned by the library (freed by
 * moe_destroy) and return its host address.  Key lE+e lives in record (lE+e) % n_records, so
 * n_records = L*E is the full pool ([FT-KR] "FreeToken의 설계": the CPU-resident pool holds
 * every routed expert; "전문가 뱅크와 FTW 포맷": banks are indexed by lE+e).  The caller fills
 * the records before the first lookup.  The memory is allocated page-locked and then filled:
 * registering already-filled memory is not used (see the design notes).
 */
MOE_API moe_status moe_pool_alloc(moe_ctx* ctx, int64_t n_records, void** host_pool);

/*
 * Use caller-owned host memory as the pool (same record indexing as moe_pool_alloc).
 * pinned = 1 promises the memory is page-locked (e.g. from hipHostMalloc); with pinned = 0 the
 * pool is pageable and only MOE_MODE_CPU may run on it (MOE_ENOPIN otherwise): every routed
 * expert then runs on the host, as in the pages' pure-CPU fallback ([FT-KR] "전문가 뱅크와
 * FTW 포맷", last paragraph).
 */
MOE_API moe_status moe_pool_register(moe_ctx* ctx, void* host_pool, int64_t n_records, int32_t pinned);
/* (Neither moe_pool_register nor moe_pool_load inspects the weights: a caller that prefills
 * FP4 / MXFP4 experts checks the pool once with moe_pool_check_f16.) */

/*
 * Bind the router weights and the slot arena.
 *  router_w: device fp32 [L, E, H].  arena: device memory of arena_bytes >= n_slots * S.
 *  n_slots:  cache slots.  MOE_MODE_FUSED needs n_slots >= L*E (slot = key; fill it with
 *            moe_fused_load).  Other modes: 0 <= n_slots <= 4096.
 * Resets the cache to empty (cold start: [FT-KR] "탄력적 메모리 관리" -- no warm-up).
 */
MOE_API moe_status moe_bind(moe_ctx* ctx, const float* router_w, void* arena, size_t arena_bytes,
                            int32_t n_slots);

/* FUSED mode: copy every pool record into arena slot = key (enqueued on stream). */
MOE_API moe_status moe_fused_load(moe_ctx* ctx, moe_stream_t stream);

/*
 * Set B_P and B_H (bytes/s) used by the q* split from now on.  Waits for all work on the
 * device.  The kernels read the slot arena, the slot count, the mode and the bandwidths from
 * a device-side control block when they run, so decode steps captured into a graph before
 * this call, moe_set_mode or expert_cache_resize follow the new values on replay.
 */
MOE_API moe_status moe_set_bandwidths(moe_ctx* ctx, uint64_t bw_pcie, uint64_t bw_host);

/*
 * Change the backend mode between steps (not FUSED <-> cached: that needs a new bind).  Waits
 * for all work on the device; captured steps follow it on replay (see moe_set_bandwidths).  A
 * step captured without a CPU branch (OFFLOAD with n_slots >= 2*T*k) whose lookup now sends
 * experts to the CPU leaves them out of y and makes the next moe_sync return MOE_ESTATE:
 * capture such steps again after the change.
 */
MOE_API moe_status moe_set_mode(moe_ctx* ctx, int32_t mode);

/*
 * Bound of a captured step's device-side wait for its CPU branch (see moe_ffn_decode), in
 * milliseconds, (0, 60000]; default 5000.  A wait that expires leaves the step's CPU experts
 * out of y and makes the next moe_sync return MOE_ETIMEDOUT.  Waits for all work on the
 * device; captured steps follow the new bound on replay.  (Failure tests make the library's
 * branch worker answer late by setting RMOE_CPU_BRANCH_DELAY_US, in microseconds, in the
 * environment before the first captured step with a CPU branch.)
 */
MOE_API moe_status moe_set_cpu_wait(moe_ctx* ctx, double timeout_ms);

/* ---- the hot path ------------------------------------------------------ */

/*
 * Router logits and top-k for T tokens of `layer` ([FT-KR] "decode 공동 설계": the router and
 * the cache lookup run on the GPU).
 *   z[t,e] = sum_h x[t,h] * W_r[layer][e,h] + logit_bias[t,e]      (fp32)
 *   topk_idx[t,:] = the k largest z[t,:], highest first, ties to the lower expert index
 *   topk_w[t,j]   = softmax(z[t,:])[topk_idx[t,j]]   (renorm = 1: divided by their sum)
 * x: device [T,H] (afmt); logit_bias: device fp32 [T,E] or NULL; logits_out: device fp32
 * [T,E] or NULL; topk_idx: device int32 [T,k]; topk_w: device fp32 [T,k].  1 <= T <= max_tokens.
 */
MOE_API moe_status moe_route(moe_ctx* ctx, int32_t layer, const void* x, int32_t T, const float* logit_bias,
                             float* logits_out, int32_t* topk_idx, float* topk_w, moe_stream_t stream);

/* The top-k and gate step of moe_route alone, on given device fp32 logits [T,E]. */
MOE_API moe_status moe_topk(moe_ctx* ctx, const float* logits, int32_t T, int32_t* topk_idx, float* topk_w,
                            moe_stream_t stream);

/*
 * One layer step of the cache control ([FT-KR] "CUDA Graph와 공존하는 LRU 캐시"; [FT-CN] 05
 * Implementation): dedupe the routed experts, classify them against the residency table, derive
 * q from the integer bandwidths (same formula as qstar_split), choose the q least recently used
 * evictable slots in one pass, admit the fills, refresh recency, and rewrite ids.
 *   topk_idx: device int32 [T,k] experts of `layer`.
 *   slot_idx: device int32 [T,k] out: slot >= 0 for GPU execution, or -1-c for entry c of the
 *             step's CPU list.
 *   trace:    device moe_trace_rec [min(T*k, E)] or NULL (one record per distinct key).
 *   counts:   device int32 [4] or NULL: hits, fills, CPU experts, evictions of occupied slots.
 * Asynchronous.  Queues the step's fill and CPU work lists for the next moe_ffn_decode of the
 * same layer.  In FUSED mode every key is a hit at slot = key and nothing changes.
 */
MOE_API moe_status expert_cache_lookup(moe_ctx* ctx, int32_t layer, const int32_t* topk_idx, int32_t T,
                                       int32_t* slot_idx, moe_trace_rec* trace, int32_t* counts,
                                       moe_stream_t stream);

/*
 * Decode expert FFN for the work of the last lookup on `layer` ([FT-KR] "측정된 대역폭이 분할을
 * 결정합니다": the CPU branch starts first; the GPU then copies the fills and evaluates the
 * resident set G = H u F; the two partial sums are added exactly):
 *   y[t] = sum_{j in G, rank order} w[t,j] FFN_{slot}(x_t) + sum_{j in C, rank order} w[t,j] FFN_key(x_t)
 * with FFN(x) = W_down (silu(W_gate x) * (W_up x)).  x: device [T,H]; topk_idx, topk_w, slot_idx
 * as given to / returned by the lookup; y: device fp32 [T,H].  Needs T * H <= 16384 (decode
 * batches); use moe_ffn_prefill for longer inputs.  Synchronises the stream when the step has
 * fills or CPU work (the fill list is read on the host), then enqueues the GPU work.
 * With MOE_FLAG_DEVICE_FILLS a cached step that cannot send work to the CPU (OFFLOAD with
 * n_slots >= 2*T*k) instead enqueues a copy kernel that executes the lookup's fill list from
 * the mapped pool ([FT-KR] "CUDA Graph와 공존하는 LRU 캐시": cache control and transfer stay
 * on the device); while `stream` is being captured, a step that may (CPU or HYBRID mode, or
 * fewer slots) also hands its CPU branch to a library thread without a host node in the
 * graph: a one-workgroup kernel writes the step block and inputs into pinned staging through
 * its device mapping and, when the lookup sent experts to the CPU, publishes a sequence
 * number in a pinned word; the thread (started by the first such step, spinning while steps
 * come, and stopped by moe_destroy) runs the branch and answers with the same number; after
 * the step's GPU experts a one-workgroup kernel polls for that answer, bounded in time (see
 * moe_set_cpu_wait), and copies the partial sum out of pinned memory for the combine.
 * Nothing is read on the calling thread, the call only enqueues work, and an out-of-range id
 * in topk_idx (the step then computes y = 0) and an expired wait are reported by the next
 * moe_sync.  Eagerly, a device-fill step that may send work to the CPU
 * queues the copy kernel behind the copies of the step block and inputs to pinned staging,
 * then the calling thread waits for those copies only, runs the CPU branch while the
 * records move, and copies its partial sum back (an out-of-range id returns MOE_EINVAL).  Needs a pool from moe_pool_alloc or a registered
 * page-locked pool with a device mapping (MOE_ENOPIN).  Such steps, and FUSED steps, may be
 * captured with route and lookup for every layer into one HIP graph on `stream` and replayed
 * (the CPU branch is served by the library thread); MOE_FLAG_PROFILE timing is skipped for captured
 * launches, and a step that would read the host while the stream is capturing returns
 * MOE_ESTATE.
 */
MOE_API moe_status moe_ffn_decode(moe_ctx* ctx, int32_t layer, const void* x, int32_t T, const int32_t* topk_idx,
                                  const float* topk_w, const int32_t* slot_idx, float* y, moe_stream_t stream);

/*
 * moe_route followed by expert_cache_lookup of the same layer and tokens, in two launches
 * instead of three: for decode-sized steps (T*k <= 64, T <= 16) the cache-control kernel
 * takes the top k from the logits itself, with the selection and gates of moe_route.
 * Arguments are those of the two calls (topk_idx and topk_w are outputs, as in
 * moe_route); the same errors.  Asynchronous on the stream.
 */
MOE_API moe_status moe_route_lookup(moe_ctx* ctx, int32_t layer, const void* x, int32_t T, const float* logit_bias,
                                    float* logits_out, int32_t* topk_idx, float* topk_w, int32_t* slot_idx,
                                    moe_trace_rec* trace, int32_t* counts, moe_stream_t stream);

/*
 * One decode layer step: moe_route_lookup, then moe_ffn_decode, with their arguments,
 * outputs and errors (y [T,H] fp32 out; topk_idx, topk_w, slot_idx [T,k] out).  In
 * MOE_MODE_FUSED at T = 1 (bf16 activations, bf16 or e2m1 weights) the lookup is the
 * identity (slot = key, group g = rank g), so phase 1 takes the top k from the logits
 * itself and the step runs in three launches (router GEMV, phase 1, the down projection
 * with the combine; four when k > 8) with results bit-identical to the two calls.
 * Asynchronous on the stream; capturable wherever moe_ffn_decode is.
 */
MOE_API moe_status moe_decode_layer(moe_ctx* ctx, int32_t layer, const void* x, int32_t T, const float* logit_bias,
                                    int32_t* topk_idx, float* topk_w, int32_t* slot_idx, float* y, moe_stream_t stream);

/*
 * Prefill over layers 0..L-1 in ascending order ([FT-KR] "전층 이중 버퍼링"; [FT-CN] 04 Design,
 * mechanism 1).  moe_prefill_begin reserves two full-layer buffers (slots [0,E) and [E,2E)) from
 * the shared pool when n_slots >= 2E and starts copying layers 0 and 1 on the library's copy
 * stream; otherwise prefill loads experts on demand.  moe_ffn_prefill(layer) waits for its layer's
 * copy, routes nothing itself (topk_idx / topk_w come from moe_route), permutes the token-expert
 * pairs by slot, runs the grouped SwiGLU GEMMs (bf16 / FP4 weights need hidden % 256 == 0 and
 * inter % 128 == 0, and bf16 weights T * hidden < 2^31, T * top_k * inter < 2^31 and records
 * below 4 GiB, else MOE_ENOTSUP), combines into y (device fp32 [T,H]) and queues the
 * copy of layer+2 into the buffer it frees.  trace (device, [min(T*k,E)] per round) and counts
 * (device int32 [4]) are optional.  moe_prefill_end returns the buffers to the pool with their
 * contents: the last two layers survive to seed decode.
 */
MOE_API moe_status moe_prefill_begin(moe_ctx* ctx, moe_stream_t stream);
MOE_API moe_status moe_ffn_prefill(moe_ctx* ctx, int32_t layer, const void* x, int32_t T, const int32_t* topk_idx,
                                   const float* topk_w, float* y, moe_trace_rec* trace, int32_t* counts,
                                   moe_stream_t stream);
MOE_API moe_status moe_prefill_end(moe_ctx* ctx, moe_stream_t stream);

/*
 * Token permutation by expert slot (a step of moe_ffn_prefill, exported on its own):
 *   perm[i]     pair index p = t*k + j of the i-th GPU pair, stably ordered by (slot, p)
 *   offsets[g]  first position of group g; offsets[n_groups] = number of GPU pairs
 *   group_slot[g] slot of group g, ascending
 * slot_idx: device int32 [T,k] (negative entries are not GPU pairs and are left out).
 * perm: device int32 [T*k]; offsets: device int32 [T*k+1]; group_slot: device int32 [T*k];
 * n_groups: device int32 [1].  Asynchronous.
 */
MOE_API moe_status moe_permute(moe_ctx* ctx, const int32_t* slot_idx, int32_t T, int32_t* perm, int32_t* offsets,
                               int32_t* group_slot, int32_t* n_groups, moe_stream_t stream);

/*
 * moe_permute for callers that cannot allocate (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): no context, no allocation, no host read.  Its
 * kernels' scratch (per-slot flags, per-pair group ids, the inverse permutation, per-chunk
 * group histograms, tile bases, counters: 2 MiB) is one array in the library's device code,
 * a copy on each device, which every call on that device shares and which keeps the last
 * call's contents: calls that overlap on one device (concurrent streams, or threads) race
 * and must be serialised by the caller.  The library looks up the array's address on a
 * device at the first call there.
 *   slot_idx     device int32 [P]: a slot id per (token, rank) pair (P = T*k, pair order
 *                t*k + j); negative entries are not GPU pairs and are left out
 *   n_slot_range every slot id must be < n_slot_range
 *   perm, offsets, group_slot  as in moe_permute: device int32 [P], [P+1], [P]
 *   n_groups     device int32 [1]: the number of groups, or -1 (the outputs are then
 *                unspecified) when a slot id is >= n_slot_range or the pairs use more than
 *                1024 distinct slots
 * Limits: 1 <= P <= 65536 and 1 <= n_slot_range <= 65536, else MOE_EINVAL (nothing is
 * enqueued).  Asynchronous on stream; MOE_EHIP if a launch fails.
 */
MOE_API moe_status moe_permute_noalloc(const int32_t* slot_idx, int32_t P, int32_t n_slot_range, int32_t* perm,
                                       int32_t* offsets, int32_t* group_slot, int32_t* n_groups,
                                       moe_stream_t stream);

/*
 * Rebuild the cache for n_slots' slots at a safe point, without touching the host pool
 * ([FT-KR] "탄력적 메모리 관리").  Shrinking keeps the n_slots' most recently used entries,
 * packed into slots 0..n_slots'-1 in ascending old-slot order (recency kept); growing adds empty
 * slots.  new_arena = NULL resizes in the bound arena (needs arena_bytes >= n_slots' * S);
 * otherwise records move to new_arena, which becomes the bound arena.  Synchronises stream, then
 * waits for all work on the device before it publishes the new arena and slot count to the
 * device-side control block the kernels read when they run: decode steps captured into a graph
 * before the resize use the resized cache on replay.  A captured step without a CPU branch
 * whose lookup finds too few slots after a shrink is reported by moe_sync (MOE_ESTATE; see
 * moe_set_mode).  MOE_ESTATE inside prefill; MOE_ENOTSUP in FUSED mode.
 */
MOE_API moe_status expert_cache_resize(moe_ctx* ctx, int32_t new_n_slots, void* new_arena, size_t new_arena_bytes,
                                       moe_stream_t stream);

/*
 * Number of misses to fill; the rest run on the CPU ([FT-KR] "측정된 대역폭이 분할을 결정합니다";
 * [FT-CN] 04 Design, mechanism 2 equations): q* = m * B_P / B_H rounded half-up, at least one
 * fill when m >= 1 and a slot is evictable, at most min(m, evictable); B_H <= B_P fills every
 * miss (the pure on-demand limit).  OFFLOAD: min(m, evictable).  CPU and FUSED: 0.
 * Negative m or evictable, or an unknown mode: returns -1.  Pure host function.
 */
MOE_API int32_t qstar_split(int32_t m, uint64_t bw_pcie, uint64_t bw_host, int32_t mode, int32_t evictable);

/*
 * Measure B_P (pinned host -> device copies of whole records) and B_H (the CPU branch over whole
 * records at batch 1) on this machine at the record size, as the pages profile both on the
 * deployed machine ([FT-KR] "실험 환경" and usage: ft bench bw).  Needs a bound pool and arena
 * with at least one slot.  Outputs bytes/s; does not change the context's bandwidths.
 */
MOE_API moe_status moe_bench_bw(moe_ctx* ctx, uint64_t* bw_pcie, uint64_t* bw_host);

/*
 * The practical HBM read rate of the current device at one transfer size: the ceiling the
 * memory-bound kernels of this library (decode GEMVs: the routed experts' records read once
 * per step; prefill GEMMs: a layer's records) are measured against.  Pass r (0 <= r < reps)
 * reads read_bytes of buf (device memory of buf_bytes, caller-owned, read only) at offset
 * (r * read_bytes) mod (buf_bytes - read_bytes + 1), rounded down to 256 bytes, with a plain
 * streaming kernel (16-byte loads, four in flight per thread), so with buf_bytes far above
 * the last-level caches every pass comes from HBM.  seconds_out[r] (host) receives pass r's
 * kernel duration.  Synchronises stream.  MOE_EINVAL: null pointers, reps < 1, read_bytes < 16
 * or above buf_bytes.
 */
MOE_API moe_status moe_bench_hbm(const void* buf, size_t buf_bytes, size_t read_bytes, int32_t reps,
                                 double* seconds_out, moe_stream_t stream);

/* Copy the residency tables to host memory (any pointer may be NULL):
 * slot_of [L*E], key_of [n_slots], stamp [n_slots]; *counter = the recency counter. */
MOE_API moe_status moe_cache_snapshot(moe_ctx* ctx, int32_t* slot_of, int32_t* key_of, uint64_t* stamp,
                                      uint64_t* counter, int32_t* n_slots);

/*
 * Wait for `stream` and report what device-fill steps could not report when they were
 * enqueued: MOE_EINVAL if a step since the last moe_sync saw an expert id out of range;
 * MOE_ESTATE if a step without a CPU branch had experts sent to the CPU by its lookup (a
 * graph captured before a shrink or a mode change; those experts are missing from y);
 * MOE_ETIMEDOUT if a captured step's wait for its CPU branch expired (see moe_set_cpu_wait).
 */
MOE_API moe_status moe_sync(moe_ctx* ctx, moe_stream_t stream);

/*
 * One layer step whose work lists the host read, logged when the context was created with
 * MOE_FLAG_PROFILE (eager decode steps that may send experts to the CPU, and steps with
 * host-issued fills): the inputs and the outcome of the q* split ([FT-KR] "측정된 대역폭이
 * 분할을 결정합니다": T_fill = q S / B_P against T_cpu for the other m - q misses).
 *   misses  m, the step's distinct routed experts not resident;  fills  q;  cpu  m - q
 *   fill_ms the fill copy of the q records: the copy kernel's duration (device fills) or the
 *           span of the host-issued copies on the copy stream; 0 when q = 0
 *   cpu_ms  wall time of the CPU branch over the cpu list; 0 when it is empty
 */
typedef struct {
  int32_t layer, misses, fills, cpu;
  double fill_ms, cpu_ms;
} moe_step_rec;

/*
 * Move up to `capacity` logged steps (oldest first) into out (host memory) and clear the log;
 * *n_out receives the number written.  Synchronises the context's streams (the fill times are
 * kernel timestamps).  At most 2^20 steps are kept between calls; later ones are dropped.
 */
MOE_API moe_status moe_step_log(moe_ctx* ctx, moe_step_rec* out, int32_t capacity, int32_t* n_out);

/* Accumulated statistics (synchronises the context's streams to read kernel timings). */
MOE_API moe_status moe_get_stats(moe_ctx* ctx, moe_stats* out);
MOE_API moe_status moe_reset_stats(moe_ctx* ctx);

/* ------------------------------------------------------------------ placement replay */

/* GPU placement policies compared on identical routing traces ([FT-KR] "무엇이 성능을 만들었나",
 * expert-locality paragraph; [FT-CN] Figure 4b; the Luce Spark post, "calibrated placement" and
 * "bounded async cache"). */
typedef enum {
  MOE_PLACE_LRU = 0,         /* the shared cache of this library, offload mode, cold start */
  MOE_PLACE_PREFILL = 1,     /* the C keys the prompt routes most, fixed for the decode */
  MOE_PLACE_STATIC = 2,      /* routing-blind: whole layers from the top, then experts 0.. below */
  MOE_PLACE_PINNED_RING = 3  /* C - L*R keys pinned by prompt frequency + an R-slot LRU ring per layer */
} moe_place_policy;

typedef struct {
  int32_t n_layers, n_experts; /* L, E */
  int32_t pairs;               /* routed (token, rank) pairs per layer step of the decode trace (T*k) */
  int32_t policy;              /* moe_place_policy */
  int32_t capacity;            /* GPU expert slots C, 0 <= C <= L*E */
  int32_t ring_per_layer;      /* PINNED_RING: R >= 0 with L*R <= C; ignored otherwise */
} moe_replay_config;

typedef struct {
  uint64_t keys;    /* distinct routed keys summed over every (step, layer) */
  uint64_t misses;  /* of those, keys not resident when their layer step began */
  uint64_t reads;   /* routed pairs (steps * L * pairs) */
} moe_replay_result;

/*
 * Replay a decode routing trace against one placement policy on the host (no GPU).  A layer
 * step's pairs are deduplicated in first-appearance order (token-major, then rank); a key misses
 * when it is not resident as the step begins.  LRU admits every miss exactly as
 * expert_cache_lookup does in MOE_MODE_OFFLOAD (victims: least recently used slots holding no
 * hit of the step; empty slots first, lowest slot first); PREFILL and STATIC never admit;
 * PINNED_RING admits an unpinned miss into its layer's ring, evicting the least recently used
 * entry that is not a hit of the step (none: not admitted).  Frequencies for PREFILL and
 * PINNED_RING count every routed pair of the calibration trace, ties to the lower key.
 *   decode     [steps][L][pairs] expert ids (host memory, caller-owned)
 *   calib      [calib_tokens][L][calib_k] expert ids of the prompt (PREFILL, PINNED_RING; else
 *              may be NULL)
 *   miss_out   NULL, or [steps][L][pairs] bytes: 1 where the pair's key missed (every pair of a
 *              missed key is marked), 0 otherwise
 * MOE_EINVAL for shapes, ids or capacities out of range.  Pure host function.
 */
MOE_API moe_status moe_placement_replay(const moe_replay_config* cfg, const int32_t* decode, int32_t steps,
                                        const int32_t* calib, int32_t calib_tokens, int32_t calib_k,
                                        uint8_t* miss_out, moe_replay_result* out);

/* ------------------------------------------------------------------ expert bank file */

/* Header of an expert bank file: the host pool stored in its runtime layout ([FT-KR]
 * "전문가 뱅크와 FTW 포맷"; [FT-CN] 05 Implementation): a 4 KiB header block, then
 * n_records records of record_bytes each in key order (key = l*E + e, or key % n_records
 * for an aliased pool), exactly the layout moe_record_bytes defines. */
typedef struct {
  int32_t n_layers, n_experts, hidden, inter, wfmt, pad;
  int64_t record_bytes, n_records;
} moe_bank_header;

typedef struct {
  uint64_t bytes;        /* record bytes read */
  double seconds;        /* wall time of the reads */
  int32_t mode;          /* 0: O_DIRECT straight into the destination; 1: O_DIRECT into per-thread
                            page-aligned buffers, then copied (destinations the kernel cannot do
                            direct I/O into); 2: buffered reads (no O_DIRECT on the file system) */
  int32_t threads;       /* reader threads */
  int32_t direct_errno;  /* errno of the first failed attempt of a faster mode, or 0 */
  int32_t pad;
} moe_bank_stats;

/* Write n_records records from `pool` (host memory, caller-owned) as a bank file for the
 * shape and format of cfg.  MOE_EINVAL for a bad shape or path, MOE_EHIP for an I/O error. */
MOE_API moe_status moe_bank_write(const char* path, const moe_config* cfg, const void* pool, int64_t n_records);

/* Read and check a bank file's header (MOE_EINVAL: missing, malformed or truncated file). */
MOE_API moe_status moe_bank_info(const char* path, moe_bank_header* out);

/*
 * Read every record of a bank file into dst (host memory of at least record_bytes *
 * n_records bytes, caller-owned) with `threads` (1..256) parallel readers in 64 MiB pieces:
 * O_DIRECT straight into dst when dst and the data size are 4 KiB-aligned and the kernel
 * accepts dst, else O_DIRECT through page-aligned per-thread buffers, else (no O_DIRECT on
 * the file system) buffered reads; `out` reports which.  cfg, when not NULL, must match the file's shape, format and
 * record size.  MOE_EINVAL for a mismatch or a short buffer, MOE_EHIP for a read error.
 * Pure host function.
 */
MOE_API moe_status moe_bank_read(const char* path, const moe_config* cfg, void* dst, int64_t dst_bytes,
                                 int32_t threads, moe_bank_stats* out);

/*
 * Engine bootstrap ([FT-KR] "탄력적 메모리 관리", fast engine bootstrap): allocate the
 * context's page-locked pool at exactly the file's record count (as moe_pool_alloc) and
 * read the bank into it; serving then starts from an empty cache, whose misses the
 * ordinary decode path fills.  The pages pin after filling; on machines that refuse to
 * page-lock existing memory the pool is allocated page-locked and filled in place.  On a
 * read error the pool is released again.  *host_pool receives the pool (owned by ctx).
 */
MOE_API moe_status moe_pool_load(moe_ctx* ctx, const char* path, int32_t threads, void** host_pool,
                                 moe_bank_stats* out);

#ifdef __cplusplus
}
#endif
#endif /* ROUTED_MOE_H */
