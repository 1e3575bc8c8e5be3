/*
 * moe.h - C ABI of the routed int4 Mixture-of-Experts layer for MI355X (gfx950).
 *
 * The layer is the one the pages are about: a GLM-5.2-shaped MoE block with
 * 256 routed experts per layer of which a router keeps 8 per token, plus one
 * always-on shared expert, with int4 expert weights (colibri summary on
 * fr.news.hada.io topic 31297, sections "Execution d'un MoE basee sur le
 * streaming disque" and "Principales fonctionnalites"; LightLX README,
 * "How it works").  Per token it computes
 *
 *   s_e   = sigmoid(x . W_r[e])                    router affinity
 *   sb_e  = s_e + bias_e                           biased score, selection only
 *   groups of E/G contiguous experts are scored by the sum of their two
 *   largest sb; the topk_group best groups stay eligible; the top_k eligible
 *   experts by sb are chosen (ties to the lower index), in sb-descending order
 *   w_j   = routed_scaling_factor * s_j / sum_chosen s
 *   d_e   = W_d,e (silu(W_g,e x) * (W_u,e x))      SwiGLU expert, no biases
 *   y     = sum_j w_j d_{e_j} + sum_shared d_s
 *
 * This is the DeepSeek-V3 "noaux_tc" sigmoid router with
 * routed_scaling_factor and a shared expert that colibri and LightLX name
 * (colibri summary, "Principales fonctionnalites"; LightLX README, "How it
 * works"), and mlx-lm's SwitchGLU expert (LightLX README, "Run any model").
 *
 * Conventions for every entry point:
 *  - Device pointers ("d_" prefix) are owned by the caller; the library never
 *    frees them and never allocates device memory, except the per-layer copy
 *    of the expert pointer table, which lives in the caller's workspace.
 *  - "stream" is a hipStream_t passed as void* (NULL = the null stream).  All
 *    GPU work is enqueued on it; calls return before the work completes
 *    unless stated otherwise.  Device faults surface at the caller's next
 *    synchronisation of that stream.
 *  - Return value: MOE_OK (0) or a negative moe_status_t.  On an argument
 *    error nothing is enqueued.  moe_last_error() describes the last failure
 *    of the calling host thread.
 *  - A handle may be used by one host thread at a time.
 */
#ifndef MOE_INT4_H
#define MOE_INT4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_EINVAL = -1,        /* bad argument or shape */
    MOE_ENOSLOT = -2,       /* expert cache: no slot can be freed right now */
    MOE_EHIP = -3,          /* a HIP runtime call failed */
    MOE_EUNSUPPORTED = -4   /* valid, but this build has no kernel for it */
} moe_status_t;

/* Layer shape.  hidden and inter are multiples of 32 (one fp16 scale per 32
 * inputs); n_experts is a multiple of n_groups; top_k <= topk_group *
 * (n_experts / n_groups).  Supported by the kernels in this build:
 * hidden/32 in {8,16,32,64,128,192,256}, inter/32 in {4,8,16,32,64,128},
 * hidden % 256 == 0, n_experts <= 256 and a multiple of 16, experts per
 * group >= 2 and a power of two times ceil(n_experts/64), n_shared in
 * {0,1}, top_k <= 8.
 * top_p in (0, 1]: adaptive expert top-p (colibri summary, options list:
 * --topp cuts the expert reads).  With top_p < 1 the selected experts are
 * ranked by their share s_j / sum_selected s (ties to the lower index), an
 * expert is kept when the shares ranked before it sum to less than top_p,
 * the kept weights are rsf * s_j / sum_kept s, and a dropped slot reports id
 * -1 and weight 0 and is never read (the batch-union dispatch gives it no
 * entry).  top_p = 1 is plain top-k. */
/* Expert weight codecs.  Both hold 32-input scale groups and two 4-bit codes
 * per byte (even column in the low nibble).
 * MOE_CODEC_INT4: two's complement int4 codes, fp16 scales (the layer's
 *   stated format).
 * MOE_CODEC_MXFP4: the GLM-5.2 MXFP4 layout that the LargerLM README streams
 *   ("What It Proves"), read as OCP MX v1.0 MXFP4: E2M1 codes (sign, 2-bit
 *   exponent with bias 1, 1-bit mantissa: 0, 0.5, 1, 1.5, 2, 3, 4, 6 and
 *   their negatives), one E8M0 scale byte b = 2^(b-127) per group (b = 255,
 *   NaN, is refused by moe_expert_pack).  19.125 MiB per expert at hidden
 *   6144, inter 2048.
 * MOE_CODEC_INT8, MOE_CODEC_INT2: the int8 and packed int2 widths of the
 *   colibri summary's quantisation kernels ("Principales fonctionnalites"),
 *   read as two's complement codes with the int4 codec's fp16 scale per 32
 *   inputs: int8 one byte per weight (code arrays [inter][hidden] and
 *   [hidden][inter]); int2 four codes per byte, column 4j + t in bits
 *   [2t, 2t + 2) of byte j (code arrays [inter][hidden/4], [hidden][inter/4]),
 *   values -2..1.
 * The batched (batch-union, matrix-core) kernels serve every codec (int2
 * where hidden is a multiple of 512 and inter of 256; other int2 T > 1 calls
 * run as T one-token passes). */
enum { MOE_CODEC_INT4 = 0, MOE_CODEC_MXFP4 = 1, MOE_CODEC_INT8 = 2, MOE_CODEC_INT2 = 3 };

typedef struct {
    int hidden;
    int inter;
    int n_experts;
    int n_groups;
    int topk_group;
    int top_k;
    int n_shared;
    float routed_scaling_factor;
    float top_p;
    int codec; /* MOE_CODEC_* (layout of the expert weights) */
} moe_config_t;

typedef struct moe_layer moe_layer_t;
typedef struct moe_cache moe_cache_t;

/* Last error message of the calling thread ("" if none). */
const char* moe_last_error(void);

/* ------------------------------------------------------------ expert weights
 * Public layout of one expert (row-major, little-endian), as on the pages'
 * int4 format with one fp16 scale per 32 inputs (colibri summary,
 * "Principales fonctionnalites": packed int4 with dequant-on-use):
 *   gate_q uint8 [inter][hidden/2]   two int4 codes per byte, two's
 *                                    complement, even column in the low nibble
 *   gate_s fp16  [inter][hidden/32]  scale of 32 consecutive input columns
 *   up_q, up_s                       as gate
 *   down_q uint8 [hidden][inter/2], down_s fp16 [hidden][inter/32]
 * Weight value = fp32(scale) * code.
 *
 * With codec MOE_CODEC_MXFP4 the codes are E2M1 and the three scale arrays
 * hold uint8 E8M0 bytes with the same shapes; MOE_CODEC_INT8 and
 * MOE_CODEC_INT2 change the code arrays' widths as above (fp16 scales).
 *
 * moe_expert_bytes: size of one packed device blob (equal to the public
 * layout's size: 3*hidden*inter * code bits / 8 + 3*hidden*inter/32 * scale
 * bytes (2, or 1 for MXFP4); for hidden 6144, inter 2048: 21,233,664 (int4),
 * 20,054,016 (MXFP4), 40,108,032 (int8), 11,796,480 (int2)).  Returns 0 for
 * an invalid config.
 *
 * moe_expert_pack: host-only repack of one expert from the public layout
 * (host pointers) into the blob format the kernels read (host buffer of
 * moe_expert_bytes bytes).  The caller copies the blob to device memory or
 * keeps it in pinned host memory for the expert cache. */
size_t moe_expert_bytes(const moe_config_t* cfg);
moe_status_t moe_expert_pack(const moe_config_t* cfg, const uint8_t* gate_q, const void* gate_s,
                             const uint8_t* up_q, const void* up_s, const uint8_t* down_q, const void* down_s,
                             void* dst_blob);

/* ------------------------------------------------------------ layer
 * moe_layer_create: d_router_w fp32 [n_experts][hidden], d_bias fp32
 * [n_experts] (the correction bias), d_shared_blobs: host array of n_shared
 * device pointers to packed shared-expert blobs.  The pointers are kept, not
 * copied: the buffers must outlive the layer.
 *
 * moe_workspace_bytes: device workspace needed for calls with up to max_T
 * tokens.  moe_layer_set_workspace: binds a caller-owned device buffer (256-
 * byte aligned), clears its control words with a synchronous memset and
 * stores the layer's expert table in it.  In all-resident mode each layer
 * needs its own workspace; layers attached to an expert cache may share one
 * when their calls are ordered on one stream.  A workspace must be bound
 * before moe_layer_set_experts.
 *
 * moe_layer_set_experts: all-resident mode.  d_blobs is a host array of
 * n_experts device pointers to packed expert blobs; the table is copied into
 * the workspace (synchronously) now if one is bound, else when one is bound.
 * A layer with an attached cache must not use this call. */
size_t moe_workspace_bytes(const moe_config_t* cfg, int max_T);
moe_status_t moe_layer_create(const moe_config_t* cfg, const float* d_router_w, const float* d_bias,
                              const void* const* d_shared_blobs, moe_layer_t** out);
moe_status_t moe_layer_set_workspace(moe_layer_t* layer, void* d_ws, size_t bytes, int max_T);
moe_status_t moe_layer_set_experts(moe_layer_t* layer, const void* const* d_blobs);
void moe_layer_destroy(moe_layer_t* layer);

/* moe_router_topk: router and group-limited top-k for T tokens.
 * d_x bf16 bits [T][hidden]; writes d_ids int32 [T][top_k] (sb descending,
 * ties to the lower index; -1 for a choice the top-p cut dropped) and d_w
 * fp32 [T][top_k] (0 for a dropped choice).  T = 0 is a no-op.  T must not
 * exceed the workspace's max_T. */
moe_status_t moe_router_topk(moe_layer_t* layer, const uint16_t* d_x, int T, int32_t* d_ids, float* d_w,
                             void* stream);

/* moe_layer_forward: the whole layer for T tokens.  d_x bf16 bits
 * [T][hidden]; d_y fp32 [T][hidden] (the block output without residual);
 * d_ids / d_w may be NULL, else receive the routing as in moe_router_topk.
 * T = 1 runs the decode kernels (three launches per token, or two, or one
 * fused launch: moe_layer_set_decode).  T > 1 runs the batch-union path for
 * every codec (colibrì summary, fr.news.hada.io topic 31297, "Principales
 * fonctionnalités implémentées": in prefill and batched verification each
 * distinct expert of the batch is read once and applied to every position
 * routed to it): routing of all tokens, a dispatch of the (token, slot)
 * entries by expert, grouped gate/up and down projections on the matrix
 * cores, and the combine; tokens are taken in launch sequences of at most
 * min(max_T, 8192 / top_k).  Int2 layers take that path where hidden is a
 * multiple of 512 and inter of 256; other int2 T > 1 calls run the decode
 * kernels token by token.  Numerics of the batched int4 calls: each weight
 * enters the matrix cores as fp16(code x scale), one rounding of at most
 * 2^-11 of itself, accumulated in fp32; this assumes every int4 group scale
 * lies in [2^-14, 2^12] (below, small codes give fp16 subnormals with fewer
 * bits; above, 8 x scale overflows fp16).  One-token calls and the other
 * codecs have no such range limit.
 * With all experts resident the call is asynchronous.  With an attached
 * expert cache the call blocks the host until the routing is known, issues
 * the copies of missing experts on the cache's copy stream and orders the
 * expert kernels after them with events: a one-token call once per token
 * (each routed expert one cache lookup, in routing order); a batched call
 * once per launch sequence, whose tokens are then taken in consecutive groups
 * (as many tokens as fit, in order, while the group's distinct experts that
 * are not pinned number at most the layer's unpinned slots) and each group's
 * distinct experts are looked up once, in ascending id order, and stay
 * resident until the group's kernels have read them. */
moe_status_t moe_layer_forward(moe_layer_t* layer, const uint16_t* d_x, int T, float* d_y, int32_t* d_ids,
                               float* d_w, void* stream);

/* moe_layer_forward_noalloc: moe_layer_forward for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops
 * and harnesses that forbid hipMalloc.  It needs no workspace (none has to be
 * bound; a bound one is not used) and allocates nothing: its per-call state
 * lives in a device array of the library, 256 KiB per GPU, held until the
 * process ends.  Same arguments and results as moe_layer_forward for an
 * all-resident layer (moe_layer_set_experts called), bit-identical to its
 * one-token calls: every token runs the decode kernels, one token after the
 * other, each call starting with one small launch that writes the expert
 * table into the array.  d_ids / d_w may be NULL.  Errors: MOE_EINVAL for a
 * layer with an expert cache or without experts, and for a shape whose
 * per-call state exceeds the array (reported with both sizes; every
 * supported shape fits).  Every call on a GPU shares that GPU's array: calls
 * that overlap on one GPU (two streams or two host threads) race; order them
 * on one stream. */
moe_status_t moe_layer_forward_noalloc(moe_layer_t* layer, const uint16_t* d_x, int T, float* d_y, int32_t* d_ids,
                                       float* d_w, void* stream);

/* moe_hbm_read_probe: device read ceiling the streaming kernels are
 * measured against (the analogue of the disk read benchmark in the colibri
 * repository, fr.news.hada.io topic 31297, "Structure du depot et
 * licence"): one launch of `blocks` workgroups of 256 threads reads the
 * `bytes` (a multiple of 16, 16-byte aligned) at d_buf once with
 * non-temporal 16-byte loads, in tiles of 32 KiB taken by the workgroups in
 * turn (each thread holds 8 loads of a tile in flight; blocks = bytes / 32 KiB
 * rounded up reads the buffer in one pass), and writes one word per
 * workgroup to d_sink (device, `blocks` words).  Asynchronous on stream;
 * time it with events.  Errors: MOE_EINVAL for a NULL pointer, a size or
 * address that is not a multiple of 16, or blocks < 1. */
moe_status_t moe_hbm_read_probe(const void* d_buf, size_t bytes, unsigned* d_sink, int blocks, void* stream);

/* moe_dispatch: the batch-union dispatch of a routing d_ids int32 [T][top_k]
 * (device) on the layer's workspace (T <= min(max_T, 8192 / top_k)):
 * d_counts [n_experts] entries per expert; d_offsets [n_experts + 1] their
 * exclusive prefix sums (d_offsets[n_experts] = the number of kept entries);
 * d_perm [T * top_k] the entries (token * top_k + slot) sorted by expert,
 * then token, then slot, followed by -1 for every id -1 (a choice the top-p
 * cut dropped, which takes no entry); d_distinct [n_experts] the experts
 * with at least one entry in ascending order, their number in
 * d_n_distinct[0] (entries of d_distinct past it are unspecified).  All
 * device buffers, asynchronous on stream.  An id outside [-1, n_experts)
 * is treated as -1 (no entry). */
moe_status_t moe_dispatch(moe_layer_t* layer, const int32_t* d_ids, int T, int32_t* d_counts, int32_t* d_offsets,
                          int32_t* d_perm, int32_t* d_distinct, int32_t* d_n_distinct, void* stream);

/* moe_layer_set_decode: how one-token calls run.  launches = 3 (the
 * default): three launches per token (router + shared gate/up, routed
 * gate/up, down + combine).  launches = 2: the router launch, then one
 * launch of co-resident workgroups that runs the routed gate/up and the down
 * projections and combine, each workgroup issuing its down weight loads
 * before it waits (inside the kernel) for every routed h.  launches = 1: one
 * fused launch per token, in which co-resident workgroups run the router,
 * the top-k, the routed and shared gate/up, the down projections and the
 * combine with the hand-offs between them done inside the kernel.  Modes 2
 * and 1 are used when their kernel has an instance for the layer's shape and
 * codec (int4 experts), the layer has no expert cache and all of the
 * launch's workgroups fit on the device at once (checked once per layer with
 * the occupancy API); otherwise three launches.  On the GLM-shaped layer
 * both take longer than the three (in one launch the waves of a CU finish
 * their gate/up work far apart and the down projections' arithmetic runs
 * after the wait instead of beside their loads), hence the default.  All
 * three give bit-identical results.  spin_limit: polls of an in-kernel wait before
 * it gives up (0: the default, about one second); a wait that gives up lets
 * the launch finish, and every later moe_layer_forward,
 * moe_layer_forward_noalloc or moe_layer_profile_read of the layer returns
 * MOE_EHIP until a workspace is bound again (moe_layer_set_workspace). */
moe_status_t moe_layer_set_decode(moe_layer_t* layer, int launches, unsigned spin_limit);

/* moe_layer_profile: when enable != 0, moe_layer_forward times each of its
 * kernel launches with HIP events on the call's stream until profiling is
 * disabled: the events are stamped with the kernel's own begin and end
 * (hipExtLaunchKernelGGL), except for the gate/up step of a layer with an
 * attached cache, whose events span the top-k launch, the wait for the
 * routing, the copies' ordering and the gate/up launches.
 * T > 1 calls on the batched kernels record kinds 0-2 as spans of their
 * stages and stamp the two grouped kernels themselves as kinds 4 and 5, and
 * the GEMV kernels of the experts with a single entry as kinds 6 and 7.
 * moe_layer_profile_read synchronises on the recorded events and returns,
 * per kind (0 router, or the batched routing + dispatch; 1 gate/up + SwiGLU
 * of the shared and routed experts, or the batched grouped gate/up + h
 * preparation; 2 down + combine, or the batched grouped down + combine; 3
 * fused one-token launch; 4 batched grouped gate/up kernel; 5 batched
 * grouped down kernel; 6 batched gate/up of single-entry experts; 7 batched
 * down of single-entry experts; 8 one-token gate/up + down launch), the
 * summed duration in milliseconds and the number of launches since
 * profiling was enabled; arrays of 9 entries.
 * Timings taken with profiling enabled are per-kernel durations, not
 * end-to-end throughput. */
moe_status_t moe_layer_profile(moe_layer_t* layer, int enable);
moe_status_t moe_layer_profile_read(moe_layer_t* layer, double* total_ms, uint64_t* launches);

/* ------------------------------------------------------------ expert cache
 * An HBM cache of packed routed experts in front of a pinned host store,
 * with one LRU per layer over a fixed set of slots (the per-layer LRU cache
 * of colibri: fr.news.hada.io topic 31297, "Execution d'un MoE basee sur le
 * streaming disque"; routed expert slots of LargerLM, "What It Proves").
 *
 * expert_cache_create: n_layers layers with slots_per_layer slots each,
 * carved from the caller's device buffer d_slot_pool of pool_bytes (at least
 * n_layers * slots_per_layer * moe_expert_bytes).  copy_stream (hipStream_t
 * as void*) carries the host-to-device copies; the cache records its own
 * events.  expert_cache_register: host blob of one routed expert, in pinned
 * host memory the caller keeps alive until destroy.  expert_cache_prefetch:
 * asynchronous copies of the listed experts into slots (no-op for resident
 * ones; MOE_ENOSLOT if every slot of the layer is held by work that has not
 * completed).  expert_cache_evict: frees the expert's slot once its last use
 * has completed (no-op MOE_OK if not resident).  expert_cache_stats: counters
 * of one layer.  moe_layer_attach_cache: routes the layer's routed experts
 * through the cache as layer layer_id.  A copy into a slot waits for every
 * earlier call's reads of it, whichever stream each call ran on; calls of
 * layers that share a workspace (and calls of one layer) are still ordered
 * by the caller. */
typedef struct {
    uint64_t hits;
    uint64_t misses;
    uint64_t h2d_bytes;
    uint64_t evictions;
    uint64_t prefetches;      /* experts copied by prefetch or pin */
    uint64_t pinned;          /* experts pinned now */
    uint64_t prefetch_hits;   /* routed uses that found an expert a prefetch brought in, unused since */
    uint64_t predicted_uses;  /* routed uses of tokens for which the previous layer predicted this layer */
    uint64_t predicted_hits;  /* of those, uses whose expert was in the prediction */
} moe_cache_stats_t;

moe_status_t expert_cache_create(const moe_config_t* cfg, int n_layers, int slots_per_layer, void* d_slot_pool,
                                 size_t pool_bytes, void* copy_stream, moe_cache_t** out);
moe_status_t expert_cache_register(moe_cache_t* cache, int layer, int expert, const void* h_pinned_blob,
                                   size_t bytes);
moe_status_t expert_cache_prefetch(moe_cache_t* cache, int layer, const int32_t* h_experts, int n);
moe_status_t expert_cache_evict(moe_cache_t* cache, int layer, int expert);
moe_status_t expert_cache_stats(const moe_cache_t* cache, int layer, moe_cache_stats_t* out);
void expert_cache_destroy(moe_cache_t* cache);
moe_status_t moe_layer_attach_cache(moe_layer_t* layer, moe_cache_t* cache, int layer_id);

/* Learning cache with a pinned hot store (colibri summary, "Learning cache
 * et attentes selon le materiel": routed experts are counted as they are
 * used, and the hottest ones are pinned in memory).
 * expert_cache_usage: copies layer's routed-use counts since creation (one
 * per expert and routed slot of every token, hits and misses alike) into
 * h_counts [n_experts].  expert_cache_pin: makes the listed experts resident
 * (copies counted as prefetches) and pins them: a pinned slot is never
 * evicted by the LRU; MOE_ENOSLOT (before any change) if the pinned experts
 * would leave fewer than top_k slots, MOE_EINVAL on an id out of range.
 * expert_cache_unpin: returns the listed experts' slots to the LRU (no-op for
 * unpinned ones).  expert_cache_autopin: unpins the layer and pins its n most
 * used experts (ties to the lower index); n must leave top_k slots.
 * expert_cache_evict frees a pinned expert's slot too. */
moe_status_t expert_cache_usage(const moe_cache_t* cache, int layer, uint64_t* h_counts);
moe_status_t expert_cache_pin(moe_cache_t* cache, int layer, const int32_t* h_experts, int n);
moe_status_t expert_cache_unpin(moe_cache_t* cache, int layer, const int32_t* h_experts, int n);
moe_status_t expert_cache_autopin(moe_cache_t* cache, int layer, int n);

/* expert_cache_replay: host-only replay of the cache's slot policy (per-layer
 * LRU; a miss takes a free slot, else the least recently used unpinned slot
 * not needed by the same token) on a routing trace [n_tokens][top_k] of one
 * layer, with no GPU work.  The n_pinned experts of `pinned` (at most
 * slots - top_k) are resident and pinned before the first token.  An id -1
 * (a choice the top-p cut dropped) is skipped, as the cache skips it.
 * Writes the hit, miss and eviction counts the cache would record for the
 * same trace from a cold start. */
moe_status_t expert_cache_replay(int n_experts, int slots, int top_k, const int32_t* trace, int n_tokens,
                                 const int32_t* pinned, int n_pinned, uint64_t* hits, uint64_t* misses,
                                 uint64_t* evictions);

/* Speculative next-layer prefetch (the expert readahead of the colibri
 * summary, "Principales fonctionnalites implementees": the next expert block
 * is fetched while the current one is being multiplied; the pages name no
 * predictor, and the one used here is the next layer's own router applied
 * to the current layer's input).
 * moe_layer_set_next: with next != NULL, every one-token call of `layer`
 * (both attached to the same expert cache, next with a bound workspace) also
 * runs next's router and top-k on this call's input, on the call's stream
 * right after this layer's router (no shared expert work, next's workspace as
 * scratch), reads the prediction back in the same host wait as this layer's
 * routing, and once this layer's own misses are queued, copies the predicted
 * experts of next that are not resident, in routing order, at most
 * max_prefetch of them (0: top_k), on the cache's copy stream.  The slot
 * choice of such a copy is a miss's, except that no predicted expert is
 * evicted for another.  next's following call counts predicted_uses /
 * predicted_hits and prefetch_hits.  next = NULL turns prediction off.
 * MOE_EINVAL if either layer has no cache, they use different caches, next
 * is layer itself, or next has no workspace or one that overlaps layer's
 * (checked again at each call).  The link is not owned: unlink (next = NULL)
 * before destroying next. */
moe_status_t moe_layer_set_next(moe_layer_t* layer, moe_layer_t* next, int max_prefetch);

/* expert_cache_replay_prefetch: expert_cache_replay with the prefetch above
 * before each token's lookup: predicted [n_tokens][top_k] holds token t's
 * prediction for this layer (a row of -1 only: no prediction for t; other
 * -1 entries are skipped), max_prefetch as in moe_layer_set_next (0:
 * top_k).  counts [7] receives hits, misses, evictions, prefetches,
 * prefetch_hits, predicted_uses, predicted_hits. */
moe_status_t expert_cache_replay_prefetch(int n_experts, int slots, int top_k, const int32_t* trace,
                                          const int32_t* predicted, int n_tokens, int max_prefetch,
                                          const int32_t* pinned, int n_pinned, uint64_t* counts);

/* Copy/compute overlap timeline of a cache.  expert_cache_timeline: with
 * enable != 0, every expert copy the cache makes (misses, prefetches, pins)
 * is bracketed by timing events on the copy stream, and every kernel that a
 * layer attached to the cache launches for a one-token call is stamped with
 * its own begin and end (unless moe_layer_profile already times it), up to
 * max_marks intervals (0: 65536; later ones are not recorded and
 * `truncated` is set); enabling clears the recorded intervals.
 * expert_cache_timeline_read synchronises on the recorded events, measures
 * the union of the copy intervals, the union of the kernel intervals and
 * their intersection (time during which a copy and a kernel both ran) over
 * the recorded window, and clears the intervals. */
typedef struct {
    double copy_ms;      /* union of the copy intervals */
    double kernel_ms;    /* union of the kernel intervals */
    double overlap_ms;   /* time with a copy and a kernel in flight */
    double span_ms;      /* first recorded begin to last recorded end */
    uint64_t copies;
    uint64_t kernels;
    int truncated;
} moe_cache_timeline_t;
moe_status_t expert_cache_timeline(moe_cache_t* cache, int enable, int max_marks);
moe_status_t expert_cache_timeline_read(moe_cache_t* cache, moe_cache_timeline_t* out);

#ifdef __cplusplus
}
#endif

#endif /* MOE_INT4_H */
