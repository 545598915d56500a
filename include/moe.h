/*
 * moe.h -- C ABI of the routed-expert FFN step on one AMD Instinct MI355X (gfx950).
 *
 * The step (LayerStoRm README, "TL;DR"): hidden states and a router go in; the
 * router picks a few experts per token; the full expert set lives in pinned host
 * RAM and GPU memory is used as a cache of experts, with the activated experts
 * streamed over PCIe and overlapped with compute; the experts' FFN outputs are
 * combined.  The GPU does all arithmetic and the host only manages the cache and
 * moves data (rebasdaily article, section "keep the experts in the warehouse").
 *
 * Conventions for every call:
 *  - Pointers are device pointers unless the name ends in _host.  The caller owns
 *    every buffer; the library owns only the moe_cache object and the hipEvents
 *    it creates.  No call allocates device memory.
 *  - `stream` arguments are hipStream_t handles passed as void* (NULL = the
 *    default stream).  Device work is enqueued asynchronously; nothing blocks
 *    except where stated.
 *  - Return value: MOE_OK (0) or a negative moe_status.  Arguments are validated
 *    before anything is enqueued, so a failed call has enqueued nothing.  A HIP
 *    runtime failure returns MOE_E_HIP and moe_last_hip_error() gives the
 *    hipError_t; moe_last_error_message() describes the last failure of the
 *    calling thread.  Device faults surface at the caller's next synchronisation.
 *  - bf16 and fp16 values are passed as uint16_t bit patterns.
 *  - Every kernel is deterministic: no floating-point atomics, fixed reduction
 *    orders, so repeated calls on the same inputs give bit-identical outputs.
 *
 * Expert slab format (one contiguous slab per expert, hidden H, intermediate I,
 * H % 32 == 0, I % 32 == 0):
 *   matrix 0 = W1 (gate) [I rows x H cols], 1 = W3 (up) [I x H], 2 = W2 (down) [H x I].
 *   A row of a matrix with K columns is K/2 code bytes (byte b holds column 2b
 *   in bits 0-3 and column 2b+1 in bits 4-7), then K/32 4-byte records, one per
 *   32-column block: fp16 scale, then fp16 min; then zero padding to a multiple
 *   of 16 bytes (none when K % 128 == 0).  Weight value = scale * code + min
 *   (exact in fp32).
 *   Slab = for r = 0..I-1 the row pair (W1 row r, W3 row r), then the H rows of
 *   W2; moe_expert_bytes(H, I) bytes (1.875 * H * I for H, I multiples of 128).
 *   Every row a kernel streams -- a gate/up pair, or a down row -- is one
 *   contiguous stretch.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
    MOE_OK = 0,
    MOE_E_ARG = -1,        /* NULL pointer, negative size, bad enum value */
    MOE_E_SHAPE = -2,      /* unsupported sizes (H or I not a multiple of 32, k > E, ...) */
    MOE_E_NOT_PINNED = -3, /* a host expert slab is not page-locked memory */
    MOE_E_NOMEM = -4,      /* caller-provided workspace or pool too small */
    MOE_E_CAPACITY = -5,   /* more experts requested at once than the cache has slots */
    MOE_E_HIP = -6,        /* a HIP runtime call failed; see moe_last_hip_error() */
    MOE_E_STATE = -7       /* call not valid in the object's current state */
} moe_status;

/* Static description of a status code. */
const char *moe_status_str(int status);
/* hipError_t behind the calling thread's last MOE_E_HIP (0 if none). */
int moe_last_hip_error(void);
/* Human-readable detail of the calling thread's last failure ("" if none). */
const char *moe_last_error_message(void);
/* Library version, e.g. 100 for 1.0.0. */
int moe_version(void);

/* Bytes of one expert slab (format above; 1.875 * hidden * inter when both are
   multiples of 128).  0 if the sizes are not positive multiples of 32. */
size_t moe_expert_bytes(int hidden, int inter);
/* Bytes of one MXFP4 expert slab (see "MXFP4 weights" below), 0 for invalid sizes. */
size_t moe_expert_bytes_mx(int hidden, int inter);
/* Bytes of one super-block expert slab (see "Super-block weights" below); 0 unless
 * hidden and inter are positive multiples of 256. */
size_t moe_expert_bytes_sb(int hidden, int inter);

/* ------------------------------------------------------------------ router
 * Router logits, top-k selection and renormalised gate weights (LayerStoRm
 * README "TL;DR": the router tells which experts a token activates;
 * glm-flash-lite page "How it works": 8 experts per layer per token).
 *   logit[t,e] = fp32( sum_h x[t,h] * w_router[e,h] + bias[e] ), products and
 *                sum in fp64, one final rounding to nearest even;
 *   topk_idx[t,:] = the k largest logits, ties to the lower expert index, in
 *                order of descending logit then ascending index;
 *   topk_w[t,i] = exp(l_i - l_0) / sum_j exp(l_j - l_0) over the k selected (fp32).
 * x [T,H] bf16 row-major; w_router [E,H] fp32 row-major; bias [E] fp32 or NULL;
 * topk_idx [T,k] int32; topk_w [T,k] fp32.  1 <= k <= min(E, 64), E <= 1024,
 * H % 32 == 0.  Inputs must be finite.
 * workspace: moe_router_workspace_bytes(T, E) bytes of device memory (contents
 * don't care; calls sharing a workspace must not overlap in time).  After the
 * call the fp32 logits [T,E] are at byte offset 256 of the workspace. */
size_t moe_router_workspace_bytes(int T, int E);
int moe_router_topk(const uint16_t *x, int T, int H, const float *w_router, const float *bias, int E,
                    int k, int32_t *topk_idx, float *topk_w, void *workspace, size_t workspace_bytes,
                    void *stream);
/* The same router for n_layers independent layers in one call (a streamed step
   routes every layer first, then plans its copies; LayerStoRm README "TL;DR":
   the router output decides what is streamed).  Layer l reads x + l*T*H,
   w_router + l*E*H, bias + l*E (bias NULL = none for every layer) and writes
   topk_idx / topk_w + l*T*k; each layer's result is bit-identical to
   moe_router_topk on that layer.  Workspace: moe_router_layers_workspace_bytes
   (n_layers, T, E) bytes; layer l's fp32 logits start at byte
   l * align_up(moe_router_workspace_bytes(T, E), 256) + 256.  n_layers <= 65535;
   n_layers == 0 or T == 0 enqueues nothing. */
size_t moe_router_layers_workspace_bytes(int n_layers, int T, int E);
int moe_router_topk_layers(const uint16_t *x, int n_layers, int T, int H, const float *w_router,
                           const float *bias, int E, int k, int32_t *topk_idx, float *topk_w, void *workspace,
                           size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------ dispatch
 * Token -> expert permutation of the T*k (token, slot) pairs p = t*k + i
 * (LayerStoRm README, "TL;DR": each token activates only the few experts the
 * router names, so a batch of tokens -- a batched decode step or a prefill chunk,
 * rebasdaily article, section "96 GB of VRAM and 208 GB of RAM behind it" -- is
 * grouped by expert so that each expert's weights are read once for all of its
 * tokens): counting sort by expert, stable in p.  count[e] = pairs routed to e;
 * offset[e] = exclusive prefix sum (offset[E] = T*k); pair_of_row[offset[e]+j] =
 * the j-th smallest pair index routed to e.  topk_idx [T,k] int32 (values in
 * 0..E-1); count [E], offset [E+1], pair_of_row [T*k] int32 outputs; all device
 * memory owned by the caller.  Requires T*k <= 16384, E <= 1024, k <= E
 * (MOE_E_SHAPE otherwise); MOE_E_ARG for a NULL pointer or T < 0; T = 0 writes
 * zero counts and offsets. */
int moe_permute(const int32_t *topk_idx, int T, int k, int E, int32_t *count, int32_t *offset,
                int32_t *pair_of_row, void *stream);

/* ------------------------------------------------------------------ expert cache
 * HBM-resident expert cache with per-layer LRU eviction, fed from pinned host RAM
 * by hipMemcpyAsync on a copy stream (LayerStoRm README "TL;DR": the full expert
 * set is pinned in host RAM, GPU memory is used as a cache, streaming overlaps
 * compute).  Per layer there are `slots_per_layer` slots of moe_expert_bytes(H,I)
 * bytes in `slot_pool` (layer l's slots start at l * slots * slab bytes).
 * expert_table: device array [n_layers * n_experts] of slab pointers (NULL = not
 * resident) the library keeps current: a layer's entries are written on the
 * compute stream by moe_cache_wait, after that layer's copies; kernels read layer
 * l's entries at expert_table + l * n_experts.  experts_host: host array
 * [n_layers * n_experts] of pinned host slab pointers.  The caller owns the
 * pool, the table and the host slabs, which must outlive the cache.
 * LRU rule per layer: a request touches its hits first (ascending expert id),
 * then its misses (ascending id); each miss evicts the least recently touched slot
 * that the same request does not need and no unreleased request holds (never-used
 * slots first, ties to the lower slot).  Not thread-safe: one host thread per cache. */
typedef struct moe_cache moe_cache;
typedef struct moe_cache_desc {
    int n_layers;
    int n_experts;
    int hidden;
    int inter;
    int slots_per_layer;
    int format; /* slab format: 0 = moe_expert_bytes slabs, 1 = MXFP4 (moe_expert_bytes_mx),
                   2 = super-blocks (moe_expert_bytes_sb) */
} moe_cache_desc;

/* Validates the description (slots <= experts), checks every host slab is pinned
   (MOE_E_NOT_PINNED otherwise), creates the events, clears expert_table with a
   blocking copy, and returns the cache in *out. */
int moe_cache_create(const moe_cache_desc *desc, const void *const *experts_host, void *slot_pool,
                     void **expert_table, void *copy_stream, moe_cache **out);
/* Query only: slot_host[i] = slot of experts_host[i] or -1, *n_hits = number resident. */
int moe_cache_lookup(moe_cache *cache, int layer, const int32_t *experts_host, int n, int32_t *slot_host,
                     int *n_hits);
/* Copy half of a prefetch.  Acquire n distinct experts of `layer` (n <= slots,
   else MOE_E_CAPACITY): touch hits, pick victims, enqueue on the copy stream each
   victim's wait for its last release and the H2D copy of each missed slab, and
   keep the layer's table writes for moe_cache_wait.  The copy stream carries only
   DMA copies and event records, so copies of several layers can be queued ahead
   of their kernels.  *n_copies (may be NULL) = misses streamed.  The acquired
   slots stay held until moe_cache_release(layer).  On a HIP failure the slots
   being filled are left empty (their experts are misses again) and the table
   writes made so far are enqueued on the copy stream at once. */
int moe_cache_prefetch_async(moe_cache *cache, int layer, const int32_t *experts_host, int n, int *n_copies);
/* Compute half: makes `compute_stream` wait for every copy of `layer` enqueued so
   far, then enqueues the layer's pending table writes on it.  A no-op when
   nothing is pending.  Call it before the kernels that read the layer's table. */
int moe_cache_wait(moe_cache *cache, int layer, void *compute_stream);
/* Splits every later slab copy into two halves, the second on
   second_copy_stream (caller-owned, default priority, same device), so that two
   DMA engines share the PCIe link: back-to-back slab-sized copies on one stream
   reach ~4% less than one large copy, two streams reach it.  The readiness and
   release ordering of moe_cache_prefetch_async / moe_cache_wait /
   moe_cache_release covers both streams.  NULL returns to one stream.
   MOE_E_STATE while a layer has copies no moe_cache_wait has covered.  A no-op
   on a recording cache. */
int moe_cache_split_copies(moe_cache *cache, void *second_copy_stream);
/* Copy timing, for measuring the link: with timing on, every later slab copy
   (each half of a split copy) is bracketed on its copy stream by two timing
   events, the first after the copy's waits for slot releases, so a copy's
   interval is the time its DMA took.  Turning timing on or off waits for the
   copies in flight and discards what was measured so far.  A no-op on a
   recording cache. */
int moe_cache_copy_timing(moe_cache *cache, int enable);
/* Waits for the copies issued so far, then reports, over the copies issued since
   timing was turned on: *busy_ms = length of the union of their intervals on
   both copy streams (the time the link was busy), *span_ms = from the first
   start to the last end, *n_copies = copies (halves) timed.  Blocks. */
int moe_cache_copy_busy(moe_cache *cache, double *busy_ms, double *span_ms, uint64_t *n_copies);
/* moe_cache_prefetch_async followed by moe_cache_wait. */
int moe_cache_prefetch(moe_cache *cache, int layer, const int32_t *experts_host, int n,
                       void *compute_stream, int *n_copies);
/* Records on `compute_stream` that every slot held by `layer` may be overwritten
   once the work enqueued so far on that stream is done, and un-holds them.
   MOE_E_STATE if the layer has copies that no moe_cache_wait has covered. */
int moe_cache_release(moe_cache *cache, int layer, void *compute_stream);
/* Cumulative hit / miss counts (per requested expert) and H2D bytes streamed. */
int moe_cache_stats(const moe_cache *cache, uint64_t *hits, uint64_t *misses, uint64_t *h2d_bytes);
/* Waits for outstanding copies and for the work enqueued before every
   moe_cache_release so far (kernels that read the slots or the table), then
   empties every slot, clears the table and zeroes the stats.  Blocks. */
int moe_cache_reset(moe_cache *cache);
/* Waits as moe_cache_reset does, then frees the library's events and the object. */
void moe_cache_destroy(moe_cache *cache);
/* Step plan of one layer (LayerStoRm README, "TL;DR": the router's choice
 * decides what is streamed; rebasdaily article, section "keep the experts in the
 * warehouse": the host manages the cache and moves the data).  ids_host: the
 * layer's n_ids top-k expert ids of the step (host memory, repeats allowed).  The
 * distinct experts are split into waves that each fit the layer's slots: one
 * wave when there are at most slots_per_layer of them; otherwise, with
 * half = max(1, slots/2) and edge = max(1, half/8), a first and a last wave of
 * edge experts and between them the fewest waves of at most half experts, sizes
 * differing by at most one (the first ones larger), taking the experts already
 * resident first and then the misses (each group in ascending id), every wave
 * sorted ascending -- so that each wave's misses can stream into slots
 * released two waves earlier while the previous wave computes, the small first
 * wave frees slots soon after the layer starts and the small last wave leaves
 * little compute after the layer's last copy.  At most ceil(n/half) + 2 waves.  Outputs (host memory): wave_experts_host [number of distinct
 * experts] the experts wave by wave; wave_start_host [max_waves + 1], wave w
 * being wave_experts_host[wave_start_host[w] .. wave_start_host[w+1]); masks_host
 * NULL or [max_waves][n_experts] uint8, set to 1 at each wave's experts and 0
 * elsewhere (the expert_mask of the wave's FFN call); *n_waves (0 when n_ids is
 * 0).  Reads the cache state only.  MOE_E_CAPACITY if more than max_waves waves
 * are needed, MOE_E_ARG for an id out of range or a NULL pointer. */
int moe_cache_plan(const moe_cache *cache, int layer, const int32_t *ids_host, int n_ids, int32_t *wave_experts_host,
                   int32_t *wave_start_host, int max_waves, uint8_t *masks_host, int *n_waves);
/* moe_cache_plan for every layer of a step in one call: ids_host [n_layers]
 * [ids_per_layer] (each layer's top-k ids); layer l's outputs at
 * wave_experts_host + l*ids_per_layer, wave_start_host + l*(max_waves+1),
 * masks_host + l*max_waves*n_experts (or NULL), n_waves_host[l].  With
 * issue_single, every layer whose experts fit its slots (one wave) is also
 * prefetched at once (moe_cache_prefetch_async of its wave), in layer order, so
 * the copy stream starts right after the plan; *n_copies (may be NULL) = the
 * misses so streamed.  Layers with several waves are left to the caller. */
int moe_cache_plan_step(moe_cache *cache, const int32_t *ids_host, int ids_per_layer, int32_t *wave_experts_host,
                        int32_t *wave_start_host, int max_waves, uint8_t *masks_host, int32_t *n_waves_host,
                        int issue_single, int *n_copies);

/* Test hook: a cache whose copy engine only records commands (no HIP calls).
   slot_pool is then just a base address used to form slot pointers.  If
   fail_copy_at > 0 the fail_copy_at-th copy reports MOE_E_HIP. */
int moe_cache_create_recording(const moe_cache_desc *desc, uintptr_t slot_pool, int fail_copy_at,
                               moe_cache **out);
/* Recorded commands of a recording cache, 4 int64 per command:
   (kind, a, b, c) with kind 1 = wait(slot, release_id, -), 2 = copy(layer, expert, slot),
   3 = table(layer, expert, slot or -1), 4 = wait(layer, -, -), 5 = release(layer, id, n_slots).
   Returns the total number of commands; writes at most max_cmds of them. */
int64_t moe_cache_trace(const moe_cache *cache, int64_t *cmds, int64_t max_cmds);

/* ------------------------------------------------------------------ expert FFN
 * Fused 4-bit block dequant + SwiGLU expert FFN for every (token, slot) pair
 * whose expert the mask admits, plus an always-on shared expert (LayerStoRm
 * README, "TL;DR": only the experts the router picks run for a token; "Serve":
 * the weights are a 4-bit block-quantised GGUF type; the 4-bit 32-column blocks
 * with an fp16 scale and min are the slab format above):
 *   g = W1 x_t, u = W3 x_t, h = bf16(silu(g) * u), y = W2 h   (fp32 accumulation)
 * x [T,H] bf16; topk_idx [T,k]; expert_table: device array [E] of this layer's
 * slab pointers (entries of masked-off experts are never read); shared_slab:
 * device slab of the shared expert or NULL; expert_mask: device uint8 [E]
 * (nonzero = compute this expert's pairs) or NULL for all.
 * y: [T*k + (shared ? T : 0), H] fp32; row t*k+i is pair (t, i), row T*k+t is the
 * shared expert for token t.  Rows of masked-off pairs are left untouched.
 * path: MOE_FFN_AUTO picks by T and k (pairs for T*k <= 64, MFMA for T >= 128,
 * split in between when H and I are multiples of 128, else grouped); the others
 * force a kernel family:
 *   MOE_FFN_PAIRS   dequant-GEMV, one group per (token, slot) pair;
 *   MOE_FFN_GROUPED dequant-GEMV, one group per expert (bit-identical to PAIRS);
 *   MOE_FFN_MFMA    grouped bf16 matrix-core kernels (weights rounded to bf16;
 *                   H and I multiples of 128);
 *   MOE_FFN_SPLIT   one group per expert: experts with up to 4 tokens on the
 *                   dequant-GEMV, the others on the MFMA kernels (H and I
 *                   multiples of 128, else as GROUPED).  The two parts run
 *                   side by side: the MFMA part on a helper stream of the
 *                   library's (one per device, created on first use), forked
 *                   from and joined back into `stream` with events, so all of
 *                   the call's work is still ordered after the work before it
 *                   on `stream` and before the work after it.
 * workspace: moe_expert_ffn_workspace_bytes(...) bytes, contents don't care. */
enum { MOE_FFN_AUTO = 0, MOE_FFN_PAIRS = 1, MOE_FFN_GROUPED = 2, MOE_FFN_MFMA = 3, MOE_FFN_SPLIT = 4 };
size_t moe_expert_ffn_workspace_bytes(int T, int H, int I, int E, int k, int has_shared);
int moe_expert_ffn(const uint16_t *x, int T, int H, int I, int E, const int32_t *topk_idx, int k,
                   const void *const *expert_table, const void *shared_slab, const uint8_t *expert_mask,
                   float *y, void *workspace, size_t workspace_bytes, int path, void *stream);

/* The two steps of moe_expert_ffn on their own, for callers that keep h or the
 * permutation themselves (and to time each kernel alone):
 *   moe_expert_gate_up: h = bf16(silu(W1 x) * (W3 x))   (dequant + gate/up + SwiGLU)
 *   moe_expert_down:    y = W2 h                         (dequant + down projection)
 * h: [T*k + (shared ? T : 0), I] bf16 with the same row numbering as y.
 * count/offset/pair_of_row: a permutation from moe_permute on the same topk_idx
 * (one kernel group per expert, weights read once per expert), or all three NULL
 * (one group per (token, slot) pair).  path: MOE_FFN_AUTO follows the presence
 * of the permutation (with it: MFMA for T >= 128, else split); MOE_FFN_GROUPED,
 * MOE_FFN_MFMA and MOE_FFN_SPLIT require it. */
int moe_expert_gate_up(const uint16_t *x, int T, int H, int I, int E, const int32_t *topk_idx, int k,
                       const int32_t *count, const int32_t *offset, const int32_t *pair_of_row,
                       const void *const *expert_table, const void *shared_slab, const uint8_t *expert_mask,
                       uint16_t *h, int path, void *stream);
int moe_expert_down(const uint16_t *h, int T, int H, int I, int E, const int32_t *topk_idx, int k,
                    const int32_t *count, const int32_t *offset, const int32_t *pair_of_row,
                    const void *const *expert_table, const void *shared_slab, const uint8_t *expert_mask,
                    float *y, int path, void *stream);

/* moe_expert_ffn, moe_expert_gate_up and moe_expert_down for expert slabs of
 * weight format `format`: 0 (the fp16 scale/min blocks above; the calls then
 * equal the ones above), 1 (MXFP4) or 2 (super-blocks), with the slab layouts of
 * the MXFP4 and super-block sections below (the pages name MXFP4 decode paths
 * among their kernels' sources: LayerStoRm README, "License and attributions";
 * their own weights are a 4-bit k-quant GGUF type: README, "Serve").  Every
 * path reads every format with the arithmetic described there; the pairs path
 * of formats 1 and 2 is the dequant-GEMV in pair grouping.  The MFMA kernels
 * form MXFP4 weights in bf16 exactly (gfx950's scaled FP4-to-bf16 convert with
 * the block's E8M0 scale) and super-block weights as format 0's (scale*q + min
 * rounded to bf16).  Super-blocks need H and I multiples of 256 (MOE_E_SHAPE);
 * automatic paths then use MFMA / split only when they are.  MOE_E_ARG for a
 * format outside 0..2. */
int moe_expert_ffn_fmt(const uint16_t *x, int T, int H, int I, int E, const int32_t *topk_idx, int k,
                       const void *const *expert_table, const void *shared_slab, const uint8_t *expert_mask,
                       float *y, void *workspace, size_t workspace_bytes, int path, int format, void *stream);
int moe_expert_gate_up_fmt(const uint16_t *x, int T, int H, int I, int E, const int32_t *topk_idx, int k,
                           const int32_t *count, const int32_t *offset, const int32_t *pair_of_row,
                           const void *const *expert_table, const void *shared_slab, const uint8_t *expert_mask,
                           uint16_t *h, int path, int format, void *stream);
int moe_expert_down_fmt(const uint16_t *h, int T, int H, int I, int E, const int32_t *topk_idx, int k,
                        const int32_t *count, const int32_t *offset, const int32_t *pair_of_row,
                        const void *const *expert_table, const void *shared_slab, const uint8_t *expert_mask,
                        float *y, int path, int format, void *stream);

/* MXFP4 on gfx950's block-scaled FP4 matrix cores (the MXFP4 decode paths the
 * pages name, LayerStoRm README, "License and attributions", with the OCP MX
 * v1.0 block scaling the hardware applies): on the MFMA path (automatic for T >=
 * 128 with H, I multiples of 128, or MOE_FFN_MFMA) moe_expert_ffn_fmt with
 * format 1 -- and so moe_mx_expert_ffn_combine / moe_mx_route_ffn_combine -- run
 * v_mfma_scale_f32_16x16x128_f8f6f4 with the slab's codes as its FP4 operand and
 * their E8M0 bytes as its scales, and no dequantisation.  Its other operand
 * takes FP8 (E4M3) values, so each bf16 activation row is first written as two
 * E4M3 digits per element, hi + lo, under one E8M0 scale 2^u per row:
 *   u = e - 8 for the row's largest magnitude f * 2^e (f in [0.5, 1));
 *   hi = x / 2^u truncated to E4M3 (3 mantissa bits; multiples of 2^-9 below
 *        2^-6), lo = x / 2^u - hi rounded to nearest-even E4M3;
 * hi + lo = x / 2^u exactly for every |x| >= 2^(u-2), i.e. within 2^10 of the
 * row's largest element (smaller ones are off by at most 2^(u-10)), so the
 * products equal those of the bf16 activations up to fp32 summation order.
 * moe_quant_act_mx does this conversion: x [rows, K] bf16 -> out [rows, 2K]
 * bytes, per 128-column group 128 hi then 128 lo bytes, each as four 32-byte
 * chunks q holding columns 16q..16q+15 then 64+16q..64+16q+15 (the operand
 * layout of lane quarter q); scales [rows] int32 = u + 127 (the E8M0 byte).
 * out may equal x (in place).  Device pointers; MOE_E_SHAPE unless K is a
 * multiple of 128 up to 16384, MOE_E_ARG for rows < 0 or NULL (rows = 0: no-op).
 * The FFN calls keep the digit pairs in their workspace (x's in the y area, h's
 * in place of h). */
int moe_quant_act_mx(const uint16_t *x, int rows, int K, uint8_t *out, int32_t *scales, void *stream);

/* Place rows computed elsewhere among the expert outputs before the combine
 * (glm-flash-lite page, "How it works": a CPU lane computes some experts beside
 * the GPU's; their rows join the GPU's): dst[rows[i],:] = src[i,:] for i < n.
 * src [n, H] fp32 (device, e.g. the CPU lane's rows uploaded in one copy); rows
 * [n] int32 (device), distinct and inside dst; dst [*, H] fp32 (device: the y of
 * moe_expert_ffn).  The caller owns every buffer.  MOE_E_ARG for n < 0, H <= 0
 * or a NULL pointer, MOE_E_SHAPE unless H % 4 == 0 and n <= 65535; n = 0 is a
 * no-op.  Rows are not checked against dst's extent (the caller's contract). */
int moe_scatter_rows(const float *src, const int32_t *rows, int n, int H, float *dst, void *stream);

/* ------------------------------------------------------------------ combine
 * Weighted combine of a token's expert outputs (LayerStoRm README, "TL;DR": the
 * selected experts' outputs are combined into the layer output; "Serve" notes: a
 * deterministic combine gives reproducible output), in a fixed order, fp32,
 * rounded once to bf16:
 *   out[t,:] = bf16( sum_{i=0..k-1} topk_w[t,i] * y[t*k+i,:] + (has_shared ? y[T*k+t,:] : 0) ).
 * y [T*k (+T), H] fp32 as produced by moe_expert_ffn; topk_w [T,k] fp32; out [T,H]
 * bf16; device memory owned by the caller.  MOE_E_ARG for T < 0, k < 1, H <= 0 or
 * a NULL pointer, MOE_E_SHAPE unless H % 4 == 0; T = 0 is a no-op. */
int moe_combine(const float *y, const float *topk_w, int T, int k, int H, int has_shared, uint16_t *out,
                void *stream);

/* Gate/up + SwiGLU, down projection and the weighted combine in one call:
 * the same arithmetic, order and roundings as moe_expert_ffn followed by
 * moe_combine, so the result is bit-identical; for a few tokens (decode) the
 * down projection and the combine run in one kernel that owns whole output
 * rows.  Every routed expert must be resident (no mask).  topk_w [T,k] fp32;
 * out [T,H] bf16; workspace: moe_expert_ffn_workspace_bytes(...). */
int moe_expert_ffn_combine(const uint16_t *x, int T, int H, int I, int E, const int32_t *topk_idx,
                           const float *topk_w, int k, const void *const *expert_table, const void *shared_slab,
                           uint16_t *out, void *workspace, size_t workspace_bytes, int path, void *stream);

/* The whole routed-expert step of one layer in one call: router (as
 * moe_router_topk) then gate/up + SwiGLU, down projection and weighted combine
 * (as moe_expert_ffn_combine), with the same arithmetic and roundings, so
 * topk_idx, topk_w and out are bit-identical to those two calls.  For one
 * token (decode) the router's last step runs inside the gate/up kernel
 * instead of a kernel of its own: three launches per layer.  Every routed
 * expert must be resident.  Arguments as in the two calls; topk_idx [T,k] and
 * topk_w [T,k] are outputs.  workspace: moe_route_ffn_combine_workspace_bytes
 * (contents don't care; calls sharing it must not overlap in time).
 * prefetch / prefetch_bytes: an optional hint, device bytes that the caller's
 * next call reads cold (e.g. the next layer's router weights, which do not
 * depend on that layer's input); for one token the down kernel reads them
 * alongside its first weight loads and discards them, so the next call finds
 * them in the device caches: 16 KB unit u is read on XCD u % 8, where the
 * router kernel's workgroup u (one expert's 16 KB of weights when H = 4096)
 * runs; as much of the hint as the kernel has waves for (1 KB per wave).
 * Results do not depend on it.  NULL and 0 for
 * none; MOE_E_ARG for a NULL pointer with a non-zero size. */
size_t moe_route_ffn_combine_workspace_bytes(int T, int H, int I, int E, int k, int has_shared);
int moe_route_ffn_combine(const uint16_t *x, int T, int H, int I, const float *w_router, const float *bias, int E,
                          int k, const void *const *expert_table, const void *shared_slab, int32_t *topk_idx,
                          float *topk_w, uint16_t *out, void *workspace, size_t workspace_bytes,
                          const void *prefetch, size_t prefetch_bytes, void *stream);

/* ------------------------------------------------------------------ chained layers
 * Residual stream between chained layers (LayerStoRm README, "Status and
 * limitations": predictive expert prefetching; "References": gating lookahead
 * behind the expert prefetch predictor; both need layer l+1's input to depend
 * on layer l's output).  The pages name no block around the MoE layers; this is
 * the plainest pre-norm residual step with the attention half left out and no
 * learned norm weight, per token row t:
 *   resid[t,:] += float(add[t,:])                    (skipped when add is NULL)
 *   x_next[t,:] = bf16_rne( resid[t,:] / sqrt(mean(resid[t,:]^2) + eps) )
 * add [T,H] bf16 (a layer's combined output) or NULL; resid [T,H] fp32, updated
 * in place; x_next [T,H] bf16, the next layer's input (must not alias add).  The
 * sum of squares is fp32 in a fixed order (reproducible run to run).  All device
 * pointers, caller-owned.  MOE_E_ARG for T < 0, H <= 0, eps outside [0, 1] or a
 * NULL resid / x_next (T = 0 is a no-op). */
int moe_residual_norm(const uint16_t *add, float *resid, int T, int H, float eps, uint16_t *x_next, void *stream);

/* ------------------------------------------------------------------ MXFP4 weights
 * A second expert weight format (the pages name MXFP4 decode paths among their
 * kernels' sources: LayerStoRm README, "License and attributions"; encodings per
 * the OCP Microscaling Formats v1.0 spec): per 32-column block 32 E2M1 codes and
 * one E8M0 scale byte v, W = E2M1(q) * 2^(v-127) (v = 255 gives NaN).  A row of K
 * columns is K/2 code bytes (byte b: column 2b in bits 0-3, 2b+1 in bits 4-7)
 * then K/32 scale bytes, zero-padded to 16 bytes; the slab holds the I row pairs
 * (W1 row r, W3 row r) then the H rows of W2, moe_expert_bytes_mx(H, I) bytes
 * (17/32 byte per weight for H, I multiples of 512).  The kernels dequantise with
 * gfx950's scaled FP4-to-bf16 convert (exact) and compute as for format 0: fp32
 * sums, h rounded once to bf16, fixed-order combine.
 *
 * One token (T = 1) with H in {2048, 4096, 6144}, I in {1536, 2048} and k +
 * shared <= 16 runs the fused one-token kernels (with the router finished inside
 * gate/up for H in {2048, 4096}); any other T or shape runs the automatic path of
 * moe_expert_ffn_fmt (pairs, split or MFMA) and moe_combine.  T = 0 is a no-op.
 * Arguments, workspace and errors otherwise as moe_expert_ffn_combine (no path
 * argument) and moe_route_ffn_combine.  A cache of MXFP4 slabs sets format = 1
 * in its descriptor. */
int moe_mx_expert_ffn_combine(const uint16_t *x, int T, int H, int I, int E, const int32_t *topk_idx,
                              const float *topk_w, int k, const void *const *expert_table, const void *shared_slab,
                              uint16_t *out, void *workspace, size_t workspace_bytes, void *stream);
int moe_mx_route_ffn_combine(const uint16_t *x, int T, int H, int I, const float *w_router, const float *bias, int E,
                             int k, const void *const *expert_table, const void *shared_slab, int32_t *topk_idx,
                             float *topk_w, uint16_t *out, void *workspace, size_t workspace_bytes,
                             const void *prefetch, size_t prefetch_bytes, void *stream);

/* ------------------------------------------------------------------ super-block weights
 * A k-quant-style format (the pages' own weights are a 4-bit k-quant GGUF
 * variant: LayerStoRm README, "TL;DR" and "Serve"; this layout is this
 * library's own): per 256-column super-block an fp16 d and fp16 dmin and, for
 * each of its eight 32-column blocks j, a 6-bit scale code s_j and a 6-bit min
 * code m_j; W = d*s_j*q - dmin*m_j for a 4-bit code q.  A K-column row (K a
 * multiple of 256) is K/2 code bytes (byte b: column 2b in bits 0-3, 2b+1 in bits
 * 4-7) then one 16-byte header per super-block: d (bytes 0-1), dmin (2-3), the
 * eight s_j (bytes 4-9) and the eight m_j (bytes 10-15), code j in bits
 * 6j..6j+5 of each 48-bit little-endian field; 4.5 bits per weight.  Same slab
 * arrangement as the other formats.  The kernels form scale d*s_j and min
 * -dmin*m_j per block (exact in fp32) and then compute as for format 0.
 * Tokens, shapes and paths as for the MXFP4 entry points (same arguments and
 * errors, plus MOE_E_SHAPE unless H and I are multiples of 256).  A cache of
 * such slabs sets format = 2 in its descriptor. */
int moe_sb_expert_ffn_combine(const uint16_t *x, int T, int H, int I, int E, const int32_t *topk_idx,
                              const float *topk_w, int k, const void *const *expert_table, const void *shared_slab,
                              uint16_t *out, void *workspace, size_t workspace_bytes, void *stream);
int moe_sb_route_ffn_combine(const uint16_t *x, int T, int H, int I, const float *w_router, const float *bias, int E,
                             int k, const void *const *expert_table, const void *shared_slab, int32_t *topk_idx,
                             float *topk_w, uint16_t *out, void *workspace, size_t workspace_bytes,
                             const void *prefetch, size_t prefetch_bytes, void *stream);

/* ------------------------------------------------------------------ CPU lane
 * Routed experts computed on host cores from the pinned host expert pool while
 * the GPU computes the others (LayerStoRm README, "Status and limitations": CPU
 * hybrid decode; glm-flash-lite page, "How it works": a GPU lane for the experts
 * in VRAM and a CPU lane for those in system RAM, side by side).  A caller sends
 * some cache misses here instead of streaming them and uploads the returned rows
 * into the y rows of their (token, expert) pairs before moe_combine.
 *
 * Per token x and expert slab: g = W1 x, u = W3 x (fp32, each 32-column block
 * as s * sum(q x) + m * sum(x), the 16 lanes of a block -- even column 2j and odd
 * column 2j+1 in lane j -- accumulated with fma across blocks and summed in a
 * fixed tree), h = bf16_rne(g / (1 + exp(-g)) * u), y = W2 h the same way (fp32).
 * Every row is computed by one thread in that fixed order: results are the same
 * for any thread count and instruction set (AVX-512, AVX2 or scalar).
 *
 * A lane owns `threads` worker threads (1..256) that run the submitted jobs in
 * order, all workers on one job at a time.  Thread-safe; the handle is the
 * caller's until moe_cpu_lane_destroy. */
typedef struct moe_cpu_lane moe_cpu_lane;
int moe_cpu_lane_create(int threads, moe_cpu_lane **out);
/* Queue one expert: slab (host memory, H, I positive multiples of 32, MOE_E_SHAPE
 * otherwise) for M tokens; x_rows[t] points at token t's H bf16 values, y_rows[t]
 * at H fp32 values the lane writes.  The lane reads the slab and the x rows until
 * the job completes (x rows are copied at submission; the slab and y rows must
 * stay valid and untouched until then).  *ticket receives the job's number;
 * M = 0 queues nothing and gives the last job's ticket.  MOE_E_ARG for a NULL
 * lane, ticket, slab or row pointer or M < 0. */
int moe_cpu_lane_submit(moe_cpu_lane *lane, const void *slab, int H, int I, int M, const uint16_t *const *x_rows,
                        float *const *y_rows, uint64_t *ticket);
/* Block until the job with this ticket and every earlier one have completed
 * (MOE_E_ARG for a ticket not yet issued). */
int moe_cpu_lane_wait(moe_cpu_lane *lane, uint64_t ticket);
/* Finish every queued job, stop the workers and free the lane (NULL: no-op). */
int moe_cpu_lane_destroy(moe_cpu_lane *lane);
/* Widest vector version this CPU runs: 512 (AVX-512), 256 (AVX2, FMA, F16C) or 0 (scalar). */
int moe_cpu_lane_isa(void);
/* Tests: run the lane with the given version (0, 256 or 512, at most
 * moe_cpu_lane_isa(); MOE_E_ARG otherwise), only with no job in flight
 * (MOE_E_STATE). */
int moe_cpu_lane_force_isa(moe_cpu_lane *lane, int isa);

/* ------------------------------------------------------------------ no allocation
 * For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): moe_route_ffn_combine
 * with its workspace in a fixed scratch array of the library instead of a
 * caller's buffer.  Same arguments (minus the workspace), arithmetic, kernels and
 * results (bit-identical), except that the split path's two parts run one after
 * the other on `stream` (no helper stream, no events).  The scratch holds
 * moe_noalloc_scratch_bytes() bytes (16 MiB) on each device, kept until the
 * process ends: calls needing a larger workspace
 * (moe_route_ffn_combine_workspace_bytes) return MOE_E_NOMEM before enqueuing
 * anything -- 32 tokens at hidden 6144, intermediate 2048, 256 experts, top-8
 * and a shared expert fit; a 2048-token chunk does not.  The call allocates
 * nothing; the first call on a device looks the array's address up.  Every call
 * on a device shares that device's array: calls that overlap in time on one
 * device (on different streams, or from different threads) race. */
size_t moe_noalloc_scratch_bytes(void);
int moe_route_ffn_combine_noalloc(const uint16_t *x, int T, int H, int I, const float *w_router, const float *bias,
                                  int E, int k, const void *const *expert_table, const void *shared_slab,
                                  int32_t *topk_idx, float *topk_w, uint16_t *out, const void *prefetch,
                                  size_t prefetch_bytes, void *stream);

/* ------------------------------------------------------------------ debug
 * Dequantise matrix `which` (0 = W1, 1 = W3, 2 = W2) of a device slab into out
 * (fp32, row-major [rows x cols]); exact, for round-trip tests of the format. */
int moe_debug_dequant(const void *slab, int H, int I, int which, float *out, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
