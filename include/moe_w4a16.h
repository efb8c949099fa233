/*
 * moe_w4a16.h -- C ABI of the MI355X (gfx950) W4A16 routed-expert MoE library.
 *
 * One MoE layer (or a residual stack of them) executed from INT4 expert
 * weights with FP16 group scales and FP16 activations:
 *   router logits -> softmax + top-k -> group tokens by expert ->
 *   gate/up projection + SwiGLU -> down projection -> weighted combine,
 * plus an optional per-layer HBM expert-slot pool for partial residency,
 * backed by an immutable pinned host copy of every expert.
 *
 * Sources (web pages):
 *   "Horizon RunMap - Architecture, Results and Public Evaluation":
 *     "Architecture invariants" (routed experts kept as INT4 with FP16 scales,
 *     FP16 activations), "What is implemented" (weights stay compact on the
 *     GPU), "The complete execution path" (route, then custom W4A16 kernels;
 *     full or partial residency), "Partial-residency contract: immutable
 *     authority and miss lifecycle" (immutable host source, H2D-only misses,
 *     publication after complete transfer, discard eviction, capacity fixed
 *     before admission, failure semantics).
 *   "An expert-offloading engine, from scratch": LRU / LFU expert caches,
 *     one contiguous blob per expert, caching never changes the output.
 *   "F51 Nitro / Nitro-MoE", "Layer 1 - expert persistence cache": slot maps,
 *     per-slot frequency and last-use counters, score freq*1000 - age, decay
 *     0.75 every 2x capacity misses, ensure() = lookup, evict, H2D, slot.
 *
 * Conventions for every call:
 *   - Pointers named "dev" are device (HBM) addresses on the context's device;
 *     "host" pointers are ordinary CPU memory.  The caller owns every buffer
 *     and stream it passes; the library owns weights, slot pools, the pinned
 *     backing, its scratch memory, its side stream and its events.
 *   - Compute calls are stream-ordered on the caller's `stream`
 *     (a hipStream_t, NULL = the null stream) and return before the GPU
 *     finishes.
 *   - Arguments are validated on the host before anything is enqueued; a
 *     failing call enqueues nothing and returns a status != MOE_OK, with text
 *     in moe_last_error().  No exception crosses the ABI.
 *   - Data-dependent problems found on the GPU (an expert id out of range or
 *     repeated within a token, an expert that is not resident in the slot
 *     pool) never cause an out-of-bounds access: the kernel substitutes a
 *     valid id or slot, computes a meaningless result for that token and
 *     sets a bit in a device error word, read by moe_check_device_errors().
 *   - One host thread per context.  Calls on one context are not thread-safe.
 *
 * Tensor layouts (all row-major, no padding):
 *   x     FP16  [T, H]          activations of the T tokens of a call
 *   ids   int32 [T, k]          selected experts of each token, rank order
 *   w     FP32  [T, k]          combine weights, same order as ids
 *   out   FP16  [T, H]          layer output
 *   h     FP32  [T, H]          residual stream of a stack
 *   q     uint8 [E][3][I*H/2]   packed INT4 codes of gate [I,H], up [I,H],
 *                               down [H,I]; row-major, element 2j of a row in
 *                               the low nibble of byte j, 2j+1 in the high one
 *   s     FP16  [E][3][I*H/128] scales: gate/up [I, H/128], down [H, I/128];
 *                               W[n,k] = (q[n,k] - 8) * s[n, k/128]
 */
#ifndef MOE_W4A16_H
#define MOE_W4A16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct moe_ctx moe_ctx; /* opaque, library-owned */

typedef enum moe_status {
  MOE_OK = 0,
  MOE_E_ARG = 1,            /* bad pointer, index or size                      */
  MOE_E_SHAPE = 2,          /* unsupported shape in moe_config                 */
  MOE_E_OOM = 3,            /* device or pinned host allocation failed         */
  MOE_E_HIP = 4,            /* a HIP runtime call failed (text has its string)  */
  MOE_E_CAPACITY = 5,       /* slot pool smaller than a routed group           */
  MOE_E_NOT_REGISTERED = 6, /* layer weights not registered yet                */
  MOE_E_TRANSFER = 7,       /* a miss transfer failed before publication       */
  MOE_E_FAULTED = 8,        /* an earlier failure after publication faulted the
                               context; only moe_destroy, moe_last_error and
                               moe_cache_stats still work                      */
  MOE_E_DEVICE = 9          /* the device error word is nonzero                */
} moe_status;

typedef enum moe_policy {
  MOE_RESIDENT_ALL = 0, /* every expert resident in HBM, no slot pool          */
  MOE_POLICY_LRU = 1,   /* evict least recently used                           */
  MOE_POLICY_LFU = 2,   /* evict least frequently used (count kept on eviction)*/
  MOE_POLICY_LRU_FREQ = 3 /* evict lowest freq*1000 - age, freq decays 0.75    */
} moe_policy;

/* Flags of moe_config.flags */
#define MOE_FLAG_ROUTER_EXACT_ALWAYS 1u /* compute every logit with the exact
                                           integer path (the certified FP64
                                           path is skipped); results are equal */
#define MOE_FLAG_FORCE_GEMV 2u          /* never take the MFMA expert path     */
#define MOE_FLAG_FORCE_MFMA 4u          /* take the MFMA path for every expert */
#define MOE_FLAG_NO_FUSED 8u            /* stacks: never take the fused one-launch
                                           decode path (use per-layer kernels)  */
#define MOE_FLAG_STAGED_TRANSPORT 16u   /* slot pools: the staged miss transport
                                           ("Horizon RunMap", "Partial-residency
                                           contract: immutable authority and miss
                                           lifecycle"): the complete host source
                                           is immutable pageable RAM, each miss
                                           goes RAM -> one of `staging_blobs`
                                           pinned staging buffers (reused once its
                                           transfer has completed) -> an
                                           unpublished spare GPU row, the routed
                                           group is published after its transfers
                                           complete, and a victim's row is reused
                                           only after the consumers of the old
                                           generation have retired (no wait for
                                           them before a copy).  Needs
                                           staging_blobs >= 1 and spare_rows >=
                                           min(C, max_tokens*k), else moe_create
                                           fails with MOE_E_CAPACITY             */

#define MOE_FLAG_GUESS_AHEAD 32u        /* stacks at batch 1 (opt-in): a kernel
                                           that loads each layer's weights during
                                           the previous layer, for the experts
                                           that layer's router picks on the
                                           previous layer's input.  The result
                                           is that of the default path within
                                           the stated tolerance.  Measured slower
                                           on MI355X than the default one-launch
                                           kernel (the weight stream slows the
                                           exchange reads of the same CUs)      */
/* Test hooks of the guess-ahead kernel, for tests of its reload path: the
 * guess of the next layer's experts is replaced by the k experts with the
 * lowest guess logits (nearly every unit's weights are loaded after the
 * selection), by the guess ranks k/2 .. k/2 + k - 1 (about half are), or by
 * no guess at all (every unit's weights are loaded after the selection).
 * The bits of the result do not depend on the guess. */
#define MOE_FLAG_TEST_GUESS_LOWEST 64u
#define MOE_FLAG_TEST_GUESS_SHIFTED 128u
#define MOE_FLAG_TEST_GUESS_NONE 256u

typedef struct moe_config {
  int32_t hidden;          /* H, multiple of 256                                  */
  int32_t n_experts;       /* E routed experts per layer, 1..1024                 */
  int32_t inter;           /* I expert intermediate size, multiple of 256         */
  int32_t top_k;           /* k, 1..16, k <= E                                    */
  int32_t renorm;          /* 1: renormalise the top-k probabilities to sum 1     */
  int32_t n_layers;        /* routed layers held by the context, >= 1            */
  int32_t shared_inter;    /* always-on shared expert intermediate (0 = none),
                              multiple of 256                                     */
  int32_t group;           /* quantisation group along K; must be 128             */
  int32_t max_tokens;      /* largest T of any call, 1..8192                      */
  int32_t device;          /* HIP device ordinal                                  */
  int32_t policy;          /* moe_policy                                          */
  int32_t slots_per_layer; /* C, slot-pool capacity per layer (policy != 0)       */
  uint32_t flags;          /* MOE_FLAG_*                                          */
  int32_t staging_blobs;   /* MOE_FLAG_STAGED_TRANSPORT: pinned staging buffers of
                              one expert blob each (context-wide)                 */
  int32_t spare_rows;      /* slot pools: GPU rows per layer beyond the C slots.
                              0 (and no staged transport): a miss is copied into
                              its victim's slot after the layer's last reader has
                              retired.  > 0: misses land in unpublished rows that
                              no generation reads, so no copy waits for the
                              current readers; a victim's row is reused only
                              after the readers of its generation retire.  Needs
                              spare_rows >= min(C, max_tokens*k) (MOE_E_CAPACITY
                              from moe_create otherwise)                          */
} moe_config;

typedef struct moe_cache_counters {
  uint64_t accesses;       /* experts requested through moe_cache_ensure          */
  uint64_t hits;
  uint64_t misses;
  uint64_t evictions;
  uint64_t h2d_bytes;      /* bytes copied host -> device for misses              */
  uint64_t d2h_bytes;      /* expert bytes copied device -> host: always 0        */
  uint64_t failures;       /* transfers that failed                               */
  double h2d_seconds;      /* side-stream busy time of completed miss and prefetch
                              copies, summed from events by moe_cache_stats
                              (syncs them)                                        */
  uint64_t prefetches;     /* experts copied by moe_cache_prefetch (also counted
                              in h2d_bytes)                                       */
  uint64_t prefetch_used;  /* prefetched copies later named by moe_cache_ensure   */
  uint64_t pinned;         /* experts of the hot set (moe_cache_pin)              */
} moe_cache_counters;

typedef struct moe_cache_event {
  int32_t step;            /* value of the ensure / prefetch call's `step`        */
  int32_t layer;
  int32_t expert;
  int32_t hit;             /* 0 miss, 1 hit, 2 prefetch fill (moe_cache_prefetch),
                              3 hit on a prefetched copy (its first use),
                              4 hot-set fill (moe_cache_pin)                      */
  int32_t slot;            /* slot the expert occupies after the call             */
  int32_t victim;          /* expert evicted from that slot, -1 if none           */
} moe_cache_event;

/* ---- lifetime -------------------------------------------------------------- */

/* Context creation ("Horizon RunMap - Architecture, Results and Public
 * Evaluation", "Partial-residency contract: immutable authority and miss
 * lifecycle": capacity is fixed before admission and a pool too small for the
 * routed group fails at startup; "The complete execution path": full or
 * partial residency of the routed experts).
 * Validates `cfg`, selects cfg->device, allocates per-layer HBM expert storage
 * (E experts, or C slots with policy != MOE_RESIDENT_ALL, plus pinned host
 * backing for all E experts), scratch sized by max_tokens, a side stream and
 * events.  Capacity is fixed here: with a slot pool, C < min(E, max_tokens*k)
 * fails with MOE_E_CAPACITY (a routed group of one call could not fit).
 * On failure *out is NULL and moe_last_error(NULL) holds the reason. */
moe_status moe_create(const moe_config* cfg, moe_ctx** out);

/* Synchronises the context's streams and frees everything it owns.  NULL is a
 * no-op. */
void moe_destroy(moe_ctx* ctx);

/* Text of the last error on `ctx` (or of the last failed moe_create when ctx is
 * NULL).  Valid until the next call on the same context. */
const char* moe_last_error(const moe_ctx* ctx);

/* ---- weights --------------------------------------------------------------- */

/* Copies one layer's weights into the library (the caller may free its arrays
 * on return).  router: host FP16 [E, H].  q, s: host arrays in the layout above.
 * shared_q [3][Is*H/2], shared_s [3][Is*H/128]: host, required iff
 * shared_inter > 0, else NULL.  The codes are re-laid in HBM (and, with a slot
 * pool, in the pinned backing) in the device tile layout; the pinned backing
 * is never written again for the context's lifetime.  Synchronous.
 * With a slot pool the layer's pool starts empty.  Re-registering a layer
 * replaces its weights (and empties its pool). */
moe_status moe_register_layer(moe_ctx* ctx, int32_t layer, const uint16_t* router,
                              const uint8_t* q, const uint16_t* s,
                              const uint8_t* shared_q, const uint16_t* shared_s);

/* ---- hot path ---------------------------------------------------------------- */

/* Router of `layer` for T tokens (1 <= T <= max_tokens) ("Horizon RunMap -
 * Architecture, Results and Public Evaluation", "The complete execution path":
 * the router picks each token's experts before the routed group is acquired;
 * "An expert-offloading engine, from scratch", "Terms used here": 8 of 64
 * experts per token; "F51 Nitro / Nitro-MoE", "The thesis": 10 of 512 plus a
 * shared expert).
 *   logit[t,e] = the FP32 value nearest (ties to even) to the exact sum
 *                sum_i x[t,i] * router[e,i];
 *   ids[t,:]   = the k experts with the largest logits, ordered by (logit
 *                descending, expert id ascending);
 *   w[t,j]     = softmax(logit[t,:])[ids[t,j]], divided by sum_j of those
 *                when cfg.renorm.
 * x: dev FP16 [T,H].  forced_ids: dev int32 [T,k] or NULL; when given,
 * selection is skipped, ids = forced_ids and w is gathered at them (ids must
 * be in range and distinct within a token, else the device error word is set).
 * ids: dev int32 [T,k] out.  w: dev FP32 [T,k] out.  logits: dev FP32 [T,E]
 * out, or NULL. */
moe_status moe_route(moe_ctx* ctx, int32_t layer, const void* x, int32_t T,
                     const int32_t* forced_ids, int32_t* ids, float* w, float* logits,
                     void* stream);

/* Routed experts of `layer` for T tokens, given their ids and weights
 * ("Horizon RunMap - Architecture, Results and Public Evaluation",
 * "Architecture invariants" and "What is implemented": the routed experts run
 * from compact INT4 data with FP16 scales and FP16 activations, never
 * expanded; "The complete execution path": custom W4A16 kernels over the
 * routed group; "An expert-offloading engine, from scratch", "Correct first":
 * caching never changes the result, hence the fixed summation order):
 *   out[t] = fp16( sum_{j=0}^{k-1} w[t,j] * FFN_{ids[t,j]}(x[t])
 *                  + FFN_shared(x[t]) )       (shared term iff shared_inter)
 *   FFN_e(x) = (silu(x Wg_e^T) * (x Wu_e^T)) Wd_e^T, silu(z) = z / (1 + e^-z),
 * with the rank-ordered sum taken in FP32 (no atomics: the result does not
 * depend on scheduling).  Expert weights are read as INT4 and never expanded
 * in HBM.  With a slot pool, every expert named in ids must have been made
 * resident by moe_cache_ensure on this layer earlier on `stream`.
 * x: dev FP16 [T,H]; ids: dev int32 [T,k]; w: dev FP32 [T,k];
 * out: dev FP16 [T,H] (must not alias x). */
moe_status moe_expert_forward(moe_ctx* ctx, int32_t layer, const void* x, int32_t T,
                              const int32_t* ids, const float* w, void* out, void* stream);

/* Allocation-free variant of moe_expert_forward, for callers that cannot
 * allocate device memory while they run it: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Same arguments,
 * results and errors as moe_expert_forward (the same kernels, bit-identical
 * outputs); the call makes no allocation of any kind (no hipMalloc, no
 * hipFree, no event or library allocation).
 * Its scratch (grouping lists, intermediates, expert outputs) lives in a
 * static array of MOE_NOALLOC_SCRATCH_BYTES in each GPU's memory, held until
 * the process ends.  A call needs about
 *   T*k*(4*H + 2*max(I, Is) + 12) + 2*T*max(I, Is) + 36*E
 *   (+ T*(2*Is + 4*H) with a shared expert)
 * bytes (each part rounded up to 256); a T that needs more returns MOE_E_ARG
 * (with the sizes in moe_last_error) and enqueues nothing.  The OLMoE-like
 * shape (H 2048, I 1024, k 8, E 64) fits up to T = 99 tokens, the
 * Qwen3-Next-like one (H 2048, I = Is = 512, k 10, E 512) up to T = 81.
 * Every call on one GPU, from any context, uses the same array: two calls
 * whose work overlaps on the GPU (different streams not ordered by events,
 * or different threads) race and give undefined results.  Nothing in the
 * array has to start at zero: every word a call reads is written earlier in
 * that call. */
#define MOE_NOALLOC_SCRATCH_BYTES (8u << 20)
moe_status moe_expert_forward_noalloc(moe_ctx* ctx, int32_t layer, const void* x, int32_t T,
                                      const int32_t* ids, const float* w, void* out, void* stream);

/* Residual stack over layers [layer_begin, layer_end):
 *   for l: x_l = fp16(RMSNorm(h)), RMSNorm(h) = h / sqrt(mean(h^2) + 1e-5);
 *          route x_l (forced_ids + l*T*k when forced_ids != NULL);
 *          h += sum_j w * FFN(x_l) (+ shared), added in FP32.
 * h: dev FP32 [T,H], updated in place.  forced_ids: dev int32 [L,T,k] indexed
 * by absolute layer, or NULL.  x_trace (dev FP16 [L,T,H]), ids_trace
 * (dev int32 [L,T,k]) and w_trace (dev FP32 [L,T,k]) receive each layer's
 * x, ids and w when non-NULL (indexed by absolute layer).  With a slot pool
 * forced_ids is required and each layer's group must have been ensured.
 * Small batches (T <= 4, T*k <= 64, T*E <= 4096, H = 2048, I in {512, 1024},
 * shared_inter in {0, I}) run as one persistent kernel per call; others run
 * the per-layer kernels.  Both give results within the stated tolerance and
 * each is deterministic.  With MOE_FLAG_GUESS_AHEAD, at T = 1 over resident
 * layers without forced_ids (and k + shared <= 12, 64 | E, E <= 512), another
 * persistent kernel loads each layer's weights during the previous layer,
 * for the experts that layer's router picks on the previous layer's input
 * ("An expert-offloading engine, from scratch", "Terms used here", "What the
 * numbers say": the next layer's experts guessed from the current state); the
 * guess changes only when weights move, never the result.  That kernel and
 * the default one may differ in the last bits of a layer's output (FP32
 * rounding of the same sums). */
moe_status moe_stack_forward(moe_ctx* ctx, int32_t layer_begin, int32_t layer_end, float* h,
                             int32_t T, const int32_t* forced_ids, void* x_trace,
                             int32_t* ids_trace, float* w_trace, void* stream);

/* The same residual stack ("Horizon RunMap", "The complete execution path"),
 * its input read from h_in: h_in (dev FP32 [T,H], read only) is the first
 * layer's residual and h (dev FP32 [T,H]) receives the result, as if h_in
 * were copied into h and moe_stack_forward ran on h.  h_in may equal h (then
 * it is moe_stack_forward); otherwise the two must not overlap
 * (MOE_E_ARG).  The one-kernel path reads h_in directly (a decode step whose
 * input sits in its own buffer needs no copy before the call); the per-layer
 * path copies it into h on `stream` first.  Other arguments, errors and
 * results as moe_stack_forward. */
moe_status moe_stack_forward_into(moe_ctx* ctx, int32_t layer_begin, int32_t layer_end, const float* h_in,
                                  float* h, int32_t T, const int32_t* forced_ids, void* x_trace,
                                  int32_t* ids_trace, float* w_trace, void* stream);

/* Synchronises `stream`, reads and clears the device error word.  Returns
 * MOE_OK if it was zero, else MOE_E_DEVICE with *bits (if non-NULL) set:
 * 1 = expert id out of range, 2 = expert repeated within a token,
 * 4 = expert not resident in the slot pool, 8 = a grid barrier of the fused
 * decode path timed out (its results are then meaningless). */
moe_status moe_check_device_errors(moe_ctx* ctx, void* stream, uint32_t* bits);

/* ---- instrumentation -------------------------------------------------------------
 * Kernel timer: while enabled for a kernel kind, every launch of that kind is
 * bracketed by a HIP event pair recorded on the stream it is launched on.
 * Kinds: 0 router logits, 1 top-k, 2 grouping, 3 gate/up + SwiGLU,
 * 4 down projection, 5 combine, 6 RMSNorm, 7 fused decode (whole stack call),
 * 8 MFMA gate/up + SwiGLU, 9 MFMA down projection (the GEMV kernels are
 * kinds 3 and 4).
 * kind = -1 disables.
 * moe_timer_read synchronises the recorded events, returns the summed
 * elapsed milliseconds and the number of launches, and resets both. */
moe_status moe_timer_enable(moe_ctx* ctx, int32_t kind);
moe_status moe_timer_read(moe_ctx* ctx, double* total_ms, int64_t* launches);

/* Phase timestamps of the fused decode path: with dev_buf (device, uint64,
 * caller-owned, at least 2*grid*stride entries) set, every block of later
 * fused launches writes the GPU's 100 MHz real-time counter at each phase
 * boundary to dev_buf[block*stride + (layer - layer_begin)*per_layer + event]
 * and its shader-clock counter at the same index + grid*stride; events
 * 0 layer start, 1 residual exchanged and normalised, 2 router logits
 * published, 3 logits exchanged, 4 selection and grouping done, 5 weight loads
 * issued, 6 gate/up published, 7 intermediates exchanged, 8 down projection
 * done, 9 residual rows published, 10 ranking done, 11 softmax done,
 * 12 down weights in LDS, 13 gate/up MFMA done, 14 gate/up partials summed.
 * Only the first 16 layers of a call are stamped; the stamps are kept on chip
 * and written when the launch ends.
 * dev_buf NULL disables.  grid, stride and per_layer (optional outputs)
 * receive the layout. */
moe_status moe_fused_phase_stamps(moe_ctx* ctx, uint64_t* dev_buf, int64_t count, int32_t* grid,
                                  int32_t* stride, int32_t* per_layer);

/* ---- expert-slot pool (partial residency) ------------------------------------ */

/* Several consumer streams on one pooled context ("Horizon RunMap -
 * Architecture, Results and Public Evaluation", "Partial-residency contract:
 * immutable authority and miss lifecycle": a request captures a generation and
 * acquires its routed group; prior-generation consumers keep their leases and
 * victim storage is reused only after they retire; the first contract
 * serialises miss transactions).  Every call of a pooled context that enqueues
 * GPU work may use its own stream.  Those calls run on the GPU one after
 * another in the order the host made them: each makes its stream wait for the
 * end of the previous one, whatever its stream, and records its own end after
 * its work.  A request -- its moe_cache_ensure calls and the compute call
 * after them, with no call of another request in between -- reads the
 * generation its ensures published.  Transfers run on the side stream
 * beside the compute of other streams: a miss lands in a row (a spare row, or
 * with in-place slots the victim's slot) only after every earlier reader of
 * that row on any stream has retired.  The host calls themselves must not
 * overlap (one thread at a time per context). */

/* ensure() of the slot pool of `layer` for one routed group ("F51 Nitro /
 * Nitro-MoE", "Layer 1 - expert persistence cache": lookup, evict, copy host
 * to device, return the slot; "Horizon RunMap - Architecture, Results and
 * Public Evaluation", "Partial-residency contract: immutable authority and
 * miss lifecycle": an all-hit group reads the existing copies, a miss is
 * transported H2D from the immutable host source and published only after
 * the transfer completes, eviction discards the GPU copy, a failure before
 * publication leaves the old generation authoritative).
 * experts: host int32 [n], distinct, 0 <= e < E, n <= C.  slots: host int32
 * [n] out: the slot each expert occupies.  step: a label copied into the event
 * log.  Hits refresh the policy state.  Each miss evicts a victim (chosen by
 * the policy among resident experts not in the group) or takes a free slot,
 * then copies the expert's blob from the pinned backing into the slot with
 * hipMemcpyAsync on the side stream, after the victim's last reader (the
 * previous compute on `stream` that used this layer) has retired.  `stream`
 * then waits for every copy of the group, and the expert->slot map in HBM is
 * updated in `stream` order, so kernels enqueued on `stream` after this call
 * see the new experts and kernels enqueued before it see the old ones.
 * Misses of one call are serialised.  A copy that fails to enqueue leaves the
 * pool and statistics as they were (MOE_E_TRANSFER); a failure after the map
 * update faults the context.  With MOE_RESIDENT_ALL: slots[i] = experts[i],
 * nothing else happens. */
moe_status moe_cache_ensure(moe_ctx* ctx, int32_t layer, const int32_t* experts, int32_t n,
                            int32_t* slots, int32_t step, void* stream);

/* Next-layer prefetch ("An expert-offloading engine, from scratch", "Terms used
 * here" and "What the numbers say": the next layer's experts are guessed by
 * running its router on the current state, and their reads start early so that
 * they overlap with computing).  experts: host int32 [n], distinct, the guessed
 * group of `layer`, n <= C.  Guessed experts already resident are left as they
 * are (no use is counted).  Each other one is filled like a miss -- lowest free
 * slot, else the policy's victim among resident experts outside the guess --
 * without a clock tick, with its LFU count unchanged, and not counted as a miss
 * (nor for the LRU-FREQ decay); its copy from the pinned backing is enqueued on
 * the side stream after the layer's last reader has retired.  Nothing is
 * published: the expert->slot map entry of a prefetched expert is written by
 * the first moe_cache_ensure that names it (after the copy completes, in that
 * call's stream order; the event log then records a hit of kind 3), and a guess
 * never used costs only its transfer and slot.  Victims' map entries are set to
 * -1 in `stream` order.  Outputs never depend on prefetching.  Returns
 * MOE_E_ARG / MOE_E_CAPACITY as moe_cache_ensure; MOE_E_TRANSFER when a copy
 * cannot be enqueued (the pool is left as it was).  With MOE_RESIDENT_ALL it
 * does nothing. */
moe_status moe_cache_prefetch(moe_ctx* ctx, int32_t layer, const int32_t* experts, int32_t n,
                              int32_t step, void* stream);

/* Residual stack with natural routing over the slot pools (partial residency):
 * for each layer l in [layer_begin, layer_end): x_l = fp16(RMSNorm(h)); route
 * layer l on x_l; when `prefetch` != 0 and l + 1 < layer_end, also route layer
 * l + 1 on x_l (the guess); read both id sets back to the host (this
 * synchronises `stream`); moe_cache_ensure(l, distinct ids of the T tokens);
 * moe_cache_prefetch(l + 1, distinct guessed ids) when the guess fits the pool's
 * dynamic slots (a guess that does not fit is not prefetched);
 * then the layer itself (as moe_stack_forward over [l, l + 1) with the routed
 * ids forced), so the guessed experts' copies run while layer l computes
 * ("An expert-offloading engine, from scratch", "What the numbers say").  The
 * result equals moe_stack_forward's with natural routing and full residency,
 * whatever is prefetched.  h: dev FP32 [T,H], updated in place; step: the
 * label of the event-log entries.  When a pinned hot set leaves fewer slots
 * than the experts of the batch's routed group outside it, the layer runs over
 * contiguous token chunks instead -- each the longest run from its first token
 * whose group fits -- ensured and computed one after another (MOE_E_CAPACITY if
 * one token's experts do not fit).  ids_trace (dev int32 [L,T,k]) receives each
 * layer's routed ids and guess_trace (dev int32 [L,T,k]) at row l + 1 the ids
 * guessed for layer l + 1, when non-NULL (indexed by absolute layer; rows not
 * written are left as they are).  Needs a slot pool (MOE_E_ARG otherwise) and
 * every layer's distinct routed experts within C (MOE_E_CAPACITY).  Returns
 * after the last layer is enqueued. */
moe_status moe_stack_forward_pooled(moe_ctx* ctx, int32_t layer_begin, int32_t layer_end, float* h,
                                    int32_t T, int32_t prefetch, int32_t step, int32_t* ids_trace,
                                    int32_t* guess_trace, void* stream);

/* Static / hybrid hot set ("An expert-offloading engine, from scratch", "What
 * the numbers say": a hot set measured on one prompt did worse than LFU on
 * another; "F51 Nitro / Nitro-MoE", "The simulator": static per-layer and
 * global hot sets against dynamic LRU).  On a cold pool (no ensure, prefetch or
 * pin on `layer` yet), the experts (host int32 [n], distinct) take slots
 * 0 .. n-1 in ascending id, are copied from the pinned backing on the side
 * stream and published in `stream` order; they are never evicted, and every
 * later group must have at most C - n experts outside the hot set
 * (MOE_E_CAPACITY from moe_cache_ensure otherwise).  The other slots stay
 * dynamic under the configured policy.  Returns MOE_E_ARG for a bad or repeated
 * id or a pool that is not cold, MOE_E_CAPACITY when n >= C, MOE_E_TRANSFER when
 * a copy cannot be enqueued (nothing changes).  With MOE_RESIDENT_ALL it does
 * nothing. */
moe_status moe_cache_pin(moe_ctx* ctx, int32_t layer, const int32_t* experts, int32_t n, int32_t step,
                         void* stream);

/* The stack's normalisation on its own: x = fp16(h / sqrt(mean(h^2) + 1e-5)),
 * unit weight, per token.  h: dev FP32 [T,H]; x: dev FP16 [T,H] out;
 * 1 <= T <= max_tokens.  Lets a caller route a layer (moe_route) before its
 * group is made resident, and guess the next layer's group from the same x. */
moe_status moe_rmsnorm(moe_ctx* ctx, const float* h, int32_t T, void* x, void* stream);

moe_status moe_cache_stats(moe_ctx* ctx, int32_t layer, moe_cache_counters* out);

/* Copies up to `cap` events of `layer` (oldest first) into buf; *n = number
 * copied.  The log keeps every event since the layer was registered. */
moe_status moe_cache_event_log(const moe_ctx* ctx, int32_t layer, moe_cache_event* buf,
                               int32_t cap, int32_t* n);

/* Test hook for the failure semantics of moe_cache_ensure, for callers that
 * test failure handling: the next call on `layer` that has misses fails
 * mode 1: before publication (as if a copy could not be enqueued; pool, policy
 * state and statistics stay as they were, MOE_E_TRANSFER), or mode 2: after
 * publication (the context is faulted, MOE_E_FAULTED).  mode 0 disarms. */
moe_status moe_debug_inject_transfer_failure(moe_ctx* ctx, int32_t layer, int32_t mode);

/* Test hook for the ordering of slot publication, for callers that test it
 * (the pages record output corrupted by an event-ordering mistake in a slot
 * cache: "F51 Nitro / Nitro-MoE", "When forced on, the cache was slower - and
 * once corrupt"): from now on every host-to-device blob copy of the context
 * is preceded on the side stream by a wait of `microseconds` (a bounded
 * kernel: it ends by the clock or, failing that, by an iteration count), so
 * a reader that does not wait for a copy's completion reads the old row.
 * Results must not change.  0 turns it off; values above
 * MOE_MAX_COPY_DELAY_US give MOE_E_ARG. */
#define MOE_MAX_COPY_DELAY_US 100000
moe_status moe_debug_delay_copies(moe_ctx* ctx, int32_t microseconds);

/* Debug mode, chosen by the environment when a context is created:
 * MOE_SYNC_EACH_CALL=1 makes every call that enqueues GPU work (moe_route,
 * moe_expert_forward and its allocation-free variant, moe_stack_forward,
 * moe_stack_forward_pooled, moe_cache_ensure, moe_cache_prefetch,
 * moe_cache_pin, moe_rmsnorm) wait for its stream and the context's side
 * stream before it returns and read the device error word: a non-zero word
 * gives MOE_E_DEVICE from that call (the word is left set; moe_check_device_errors
 * reads and clears it).  Not for use under stream capture. */

/* ---- host-only policy engine (no device needed) --------------------------------
 * The decision procedure moe_cache_ensure uses, exposed on its own so it can be
 * exercised without a GPU.  Per call: the clock ticks; the group (processed in
 * ascending id) first refreshes its hits, then fills each miss from the lowest
 * free slot or evicts the resident expert outside the group with the smallest
 * key -- LRU (last, id); LFU (count, last, id); LRU-FREQ
 * (sfreq*1000 - (clock - last), id) in double, sfreq = 1 on fill, +1 per hit,
 * all sfreq *= 0.75 after every 2*C misses.  Events are appended hits first,
 * then misses, each in ascending id. */
typedef struct moe_policy_engine moe_policy_engine;

moe_policy_engine* moe_policy_new(int32_t policy, int32_t n_experts, int32_t capacity,
                                  int32_t layer);
void moe_policy_free(moe_policy_engine* p);
/* Returns MOE_OK, MOE_E_ARG (bad id, repeated id) or MOE_E_CAPACITY (n > C).
 * slots [n] out in the order of `experts`; events appended to the engine's log. */
moe_status moe_policy_access(moe_policy_engine* p, const int32_t* experts, int32_t n,
                             int32_t step, int32_t* slots);
/* The decision part of moe_cache_pin (MOE_E_ARG for a pool that is not cold). */
moe_status moe_policy_pin(moe_policy_engine* p, const int32_t* experts, int32_t n, int32_t step);
/* The decision part of moe_cache_prefetch (same rules and return codes). */
moe_status moe_policy_prefetch(moe_policy_engine* p, const int32_t* experts, int32_t n,
                               int32_t step);
int32_t moe_policy_event_count(const moe_policy_engine* p);
int32_t moe_policy_events(const moe_policy_engine* p, moe_cache_event* buf, int32_t cap);

/* ---- offline routing-trace analysis (host only, no device needed) -------------
 * Captured router traces replayed through cache policies offline, hit rate per
 * capacity ("F51 Nitro / Nitro-MoE", "The simulator"); LRU against LFU at a fixed
 * cache size ("An expert-offloading engine, from scratch", "What the numbers
 * say"); the share a static pin of the most popular experts serves ("F51 Nitro /
 * Nitro-MoE", "Layer 1 - expert persistence cache").
 *
 * A trace is one layer's routed groups: `ids` host int32 row-major
 * [n_steps, width], read only, owned by the caller.  An entry < 0 is padding; an
 * expert named twice in one row counts once; an entry >= n_experts is
 * MOE_E_ARG.  Nothing is kept after the call returns. */

/* Belady's rule for groups: every expert of a step's group must be resident at
 * once; a miss takes a free slot, else evicts the resident expert outside the
 * group whose next use is farthest (never again = infinitely far; ties to the
 * lower id).  Hits of a step are counted before its misses are filled.
 * hits/misses out.  MOE_E_CAPACITY when a group has more than `capacity`
 * distinct experts. */
moe_status moe_trace_opt(const int32_t* ids, int32_t n_steps, int32_t width, int32_t n_experts,
                         int32_t capacity, int64_t* hits, int64_t* misses);
/* The online policy (MOE_POLICY_LRU / _LFU / _LRU_FREQ) of moe_cache_ensure,
 * one access per row (the same engine as moe_policy_access). */
moe_status moe_trace_policy(int32_t policy, const int32_t* ids, int32_t n_steps, int32_t width,
                            int32_t n_experts, int32_t capacity, int64_t* hits, int64_t* misses);
/* moe_trace_policy with the hot set `hot` (host int32 [n_hot], distinct) pinned
 * first, as moe_cache_pin does: those experts are never evicted and count as
 * hits whenever named; the other capacity - n_hot slots run the policy.
 * MOE_E_CAPACITY when n_hot >= capacity or a row has more than
 * capacity - n_hot experts outside the hot set. */
moe_status moe_trace_policy_pinned(int32_t policy, const int32_t* ids, int32_t n_steps, int32_t width,
                                   int32_t n_experts, int32_t capacity, const int32_t* hot, int32_t n_hot,
                                   int64_t* hits, int64_t* misses);
/* Share of all selections (selection = a row naming an expert) that fall on the
 * n_top most-selected experts, ties to the lower id: the hit rate of a static
 * pin of those experts.  0 for an empty trace. */
moe_status moe_trace_top_share(const int32_t* ids, int32_t n_steps, int32_t width, int32_t n_experts,
                               int32_t n_top, double* share);
typedef struct moe_skew_report {
  double top10, top20, top30;  /* top shares of ceil(p*E) experts, p = 10/20/30 %   */
  double entropy_bits;         /* entropy of the selection frequencies (log2)       */
  int32_t distinct;            /* experts selected at least once                    */
  int64_t selections;          /* all selections                                    */
} moe_skew_report;
moe_status moe_trace_skew(const int32_t* ids, int32_t n_steps, int32_t width, int32_t n_experts,
                          moe_skew_report* out);

#ifdef __cplusplus
}
#endif
#endif /* MOE_W4A16_H */
