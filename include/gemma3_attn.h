/*
 * gemma3_attn.h -- C ABI of the MI355X (gfx950) Gemma 3 attention-block forward.
 *
 * What it computes (study-note pages on Gemma 3):
 *   "Gemma 3 Attention Block", How it works: Q = q_einsum(x), K,V = kv_einsum(x);
 *     RMSNorm on Q and on K, then RoPE with the layer's (theta, scale), then the
 *     query scale alpha; grouped scores sum_c Q[t,h,c] K[s,h/G,c]; causal and
 *     padding mask, times the sliding mask 1[s > t-W] 1[s < t+W] on local
 *     layers, blocked entries filled with K_MASK = -2.3819763e38; softmax over
 *     s; weights mix V; attn_vec_einsum maps heads back to D. A decode step
 *     writes the new K and V into a left-aligned cache and attends to it.
 *   "QK-Norm", How it works: RMSNorm(v) = v / sqrt(mean(v^2) + 1e-6) * (1 + gamma)
 *     over the head dimension, separate gammas for Q and K, V not normalised,
 *     applied before RoPE; alpha applied after RoPE.
 *   "Global vs Local Layer Routing", How it works: layer l has type
 *     P[l mod 6] with P = (L, L, L, L, L, G); local layers use theta = 1e4,
 *     scale 1 and the window; global layers theta = 1e6 and scale 8 (or 1 on
 *     the 1B/270M sizes). This ABI takes the resolved (type, W, theta, scale).
 *
 * Conventions fixed by this library (the pages leave them open):
 *   - RoPE pairs channel i with channel i + d_h/2; channel pair i turns by
 *     (pos / scale) * theta^(-2i/d_h) radians: (a, b) -> (a cos - b sin, b cos + a sin).
 *   - gamma_q, gamma_k are [d_h] vectors shared by every head and position.
 *   - Query head h reads KV head h / G, G = H / H_kv.
 *   - Prefill masks use token indices (t, s); segment_pos only feeds RoPE.
 *     Key s of batch row b is padding when s >= kv_valid_len[b].
 *   - Decode: cache slot s holds position s (left-aligned); the query of row b
 *     sits at pos_b = segment_pos[b] and its rotated key and its value are
 *     written to slot pos_b before attending to slots s <= pos_b (and
 *     s > pos_b - W on local layers).
 *   - A row with no allowed key outputs 0 instead of the fill-value result
 *     (uniform mean over all keys). Causal masking alone never produces one
 *     (key t is allowed); padding does when kv_valid_len[b] == 0, or on a
 *     local layer for rows t >= kv_valid_len[b] + W - 1 (a padded tail
 *     longer than the window).
 *
 * Layouts (all row-major, element type per desc.dtype):
 *   x            [B, T, D]
 *   segment_pos  [B, T] int32                      (device)
 *   kv_valid_len [B] int32 or NULL = all T valid   (device)
 *   w_q          [H*d_h, D]       output-major: row h*d_h + c is head h, channel c
 *   w_kv         [2*H_kv*d_h, D]  rows 0..H_kv*d_h-1 are K heads, then V heads
 *   w_o          [D, H*d_h]       y[., j] = sum_n o[., n] * w_o[j, n]
 *   gamma_q, gamma_k [d_h]
 *   y            [B, T, D]
 *   k_cache, v_cache [B, S, H_kv, d_h]  (decode only)
 *
 * Ownership and threading: every pointer is a DEVICE pointer unless noted;
 * the caller owns every buffer, the library allocates nothing, keeps no
 * pointer after it returns and holds no global state (the one exception is
 * the static scratch of gemma3_attn_decode_static, described there). Work is enqueued on
 * `hip_stream` (a hipStream_t, NULL = the default stream) and the call
 * returns without synchronising; buffers must stay alive until the stream
 * passes the work. y must not alias an input; the workspace must not alias
 * anything else. Calls on different streams need different workspaces.
 *
 * Errors: every call returns a gemma3_status. All host-side validation runs
 * before the first enqueue, so on any status other than GEMMA3_OK and
 * GEMMA3_ERR_HIP nothing was enqueued. GEMMA3_ERR_HIP means a launch failed
 * (outputs undefined). The library never aborts, prints or synchronises.
 * Preconditions on device data that the host cannot see without a sync:
 * 0 <= kv_valid_len[b] <= T, 0 <= segment_pos[b] < S in decode; a decode
 * position outside [0, S) makes that row skip its cache write and output 0.
 */
#ifndef GEMMA3_ATTN_H
#define GEMMA3_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GEMMA3_ATTN_ABI_VERSION 3

/* AttentionType ("Global vs Local Layer Routing", How it works). */
typedef enum { GEMMA3_ATTN_GLOBAL = 0, GEMMA3_ATTN_LOCAL_SLIDING = 1 } gemma3_attn_type;

/* Element type of x, weights, gammas, y and the cache. Accumulation is fp32. */
typedef enum { GEMMA3_F32 = 0, GEMMA3_BF16 = 1 } gemma3_dtype;

typedef enum {
  GEMMA3_OK = 0,
  GEMMA3_ERR_NULL = 1,        /* a required pointer is NULL */
  GEMMA3_ERR_SHAPE = 2,       /* non-positive size, H % H_kv != 0, odd d_h, T != 1 in decode */
  GEMMA3_ERR_WINDOW = 3,      /* local layer with window < 1 */
  GEMMA3_ERR_DTYPE = 4,       /* unknown dtype or attention type */
  GEMMA3_ERR_ROPE = 5,        /* theta <= 0, scale <= 0, or a non-finite theta/scale/alpha */
  GEMMA3_ERR_WORKSPACE = 6,   /* workspace NULL or smaller than gemma3_attn_workspace_bytes */
  GEMMA3_ERR_UNSUPPORTED = 7, /* valid shape this library has no kernel for (see below) */
  GEMMA3_ERR_HIP = 8,         /* a kernel launch failed */
  GEMMA3_ERR_ALIGN = 9,       /* a pointer is not 16-byte aligned */
  GEMMA3_ERR_SCRATCH = 10     /* workspace need exceeds GEMMA3_STATIC_SCRATCH_BYTES (static entry points) */
} gemma3_status;

/* One attention layer. All sizes are element counts. */
typedef struct {
  int32_t B, T, D, H, H_kv, d_h; /* T == 1 for decode; H % H_kv == 0; d_h even */
  int32_t attn_type;             /* gemma3_attn_type */
  int32_t window;                /* W >= 1 when LOCAL_SLIDING; ignored when GLOBAL */
  float rope_theta;              /* theta > 0 */
  float rope_scale;              /* > 0; RoPE positions are divided by it */
  float query_scale;             /* alpha (e.g. d_h^-1/2, or (D/H)^-1/2 for 27B shapes), finite */
  int32_t dtype;                 /* gemma3_dtype */
} gemma3_attn_desc;

/* Weights of one layer (device pointers, layouts above, element type dtype). */
typedef struct {
  const void *w_q;
  const void *w_kv;
  const void *w_o;
  const void *gamma_q;
  const void *gamma_k;
} gemma3_attn_weights;

/*
 * Shapes with kernels in this library:
 *   GEMMA3_BF16: d_h in {64, 128, 256}; D % 64 == 0; H*d_h % 64 == 0;
 *                B*T < 2^31 / max(D, (H + 2 H_kv) d_h).
 *   GEMMA3_F32:  d_h in {16, 32, 64, 128, 256}; any D, H, H_kv, B, T within int32.
 *   Decode (both dtypes): d_h a multiple of 64.
 * Anything else valid returns GEMMA3_ERR_UNSUPPORTED.
 */

/* Bytes of device workspace prefill (S == 0) or decode (S = cache length)
 * needs for this descriptor; 0 when the descriptor is invalid. */
size_t gemma3_attn_workspace_bytes(const gemma3_attn_desc *desc, int32_t S);

/*
 * Prefill: y = Attention(x) for every token of every row, no cache
 * ("Gemma 3 Attention Block", How it works, S = T). Masks: causal on token
 * indices, keys s >= kv_valid_len[b] blocked, and on local layers keys
 * s <= t - W blocked. segment_pos feeds RoPE only.
 */
int gemma3_attn_prefill(const gemma3_attn_desc *desc, const void *x,
                        const int32_t *segment_pos, const int32_t *kv_valid_len,
                        const gemma3_attn_weights *w, void *y, void *workspace,
                        size_t workspace_bytes, void *hip_stream);

/*
 * Prefill that also fills a left-aligned cache ("Gemma 3 Attention Block",
 * How it works, Cache: the call's keys and values are written into a
 * left-aligned buffer of S slots). Computes y exactly as gemma3_attn_prefill
 * does (the attention sees the T tokens of this call only), then writes the
 * rotated key and the value of every valid token t (t < kv_valid_len[b], or
 * every t when kv_valid_len is NULL) of every KV head to slot
 * segment_pos[b*T + t] of k_cache and v_cache: device arrays
 * [B, S, H_kv, d_h] of the descriptor's dtype (the layout gemma3_attn_decode
 * reads), 16-byte aligned, owned by the caller. Tokens whose position lies
 * outside [0, S) and every other slot are left untouched. Positions within a
 * row should be distinct: when two tokens share a slot, either may end up
 * there. The workspace is the prefill's (gemma3_attn_workspace_bytes(desc, 0)).
 * Errors: those of gemma3_attn_prefill; S < 1 -> GEMMA3_ERR_SHAPE; a NULL
 * cache -> GEMMA3_ERR_NULL; a misaligned cache -> GEMMA3_ERR_ALIGN. Nothing
 * is enqueued when an error is returned before the first launch.
 */
int gemma3_attn_prefill_cache(const gemma3_attn_desc *desc, const void *x,
                              const int32_t *segment_pos, const int32_t *kv_valid_len,
                              const gemma3_attn_weights *w, void *k_cache, void *v_cache,
                              int32_t S, void *y, void *workspace, size_t workspace_bytes,
                              void *hip_stream);

/*
 * Prefill chunk: continues rows whose first `start` tokens are already in
 * the left-aligned cache ("Gemma 3 Attention Block", How it works: the
 * prefill steps, with the Cache passage's slot = position). The T tokens of
 * x have indices start .. start+T-1 and segment_pos[b*T + t] should equal
 * start + t (it feeds RoPE and names the slot written). Their rotated keys
 * and values are written to the cache as gemma3_attn_prefill_cache does;
 * then every query attends to cache slots 0 .. start+T-1 under the causal
 * and padding masks (and the window on local layers) of one prefill over the
 * whole sequence: keys at or past start + kv_valid_len[b] are blocked
 * (start + T without kv_valid_len). Slots 0 .. start-1 must hold the rows'
 * earlier keys and values (from gemma3_attn_prefill_cache, earlier chunks or
 * decode steps). With start = 0 this is gemma3_attn_prefill_cache.
 * Caches: [B, S, H_kv, d_h] device arrays of the descriptor's dtype,
 * 16-byte aligned, start + T <= S. The attention reads the keys and values
 * in the caches where they are (slots at or past start + kv_valid_len[b] are
 * never used, whatever they hold). Workspace:
 * gemma3_attn_prefill_chunk_workspace_bytes(desc, start) bytes; the size
 * does not depend on start (the argument is only validated: < 0 -> 0).
 * Errors: those of gemma3_attn_prefill; start < 0, S < 1 or start + T > S ->
 * GEMMA3_ERR_SHAPE; a NULL cache -> GEMMA3_ERR_NULL; misaligned ->
 * GEMMA3_ERR_ALIGN; a short workspace -> GEMMA3_ERR_WORKSPACE.
 */
size_t gemma3_attn_prefill_chunk_workspace_bytes(const gemma3_attn_desc *desc, int32_t start);
int gemma3_attn_prefill_chunk(const gemma3_attn_desc *desc, const void *x,
                              const int32_t *segment_pos, const int32_t *kv_valid_len,
                              const gemma3_attn_weights *w, void *k_cache, void *v_cache,
                              int32_t S, int32_t start, void *y, void *workspace,
                              size_t workspace_bytes, void *hip_stream);

/*
 * Decode: one token per row against a left-aligned cache of S slots
 * ("Gemma 3 Attention Block", How it works, Cache). Writes the rotated key
 * and the value of row b into k_cache/v_cache slot segment_pos[b], then
 * attends to slots 0..segment_pos[b] (global) or the last W of them (local).
 * Slots past segment_pos[b] are never read (they may hold anything, NaN included).
 */
int gemma3_attn_decode(const gemma3_attn_desc *desc, const void *x,
                       const int32_t *segment_pos, const gemma3_attn_weights *w,
                       void *k_cache, void *v_cache, int32_t S, void *y,
                       void *workspace, size_t workspace_bytes, void *hip_stream);

/*
 * Allocation-free decode, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): gemma3_attn_decode with the same arguments, results and errors,
 * but no workspace argument. Its workspace is a static device array of
 * GEMMA3_STATIC_SCRATCH_BYTES in the library, one copy per GPU, set up by
 * the first call on that GPU (with the caller's current device, which must
 * be the device of hip_stream) and held until the process ends; the call
 * itself allocates nothing. Shapes whose decode workspace
 * (gemma3_attn_workspace_bytes(desc, S)) exceeds it return
 * GEMMA3_ERR_SCRATCH and enqueue nothing (the 12B-like step, B = 16,
 * S = 131072, needs 36.5 MiB). Every call on one GPU shares that GPU's
 * array and nothing in it needs to start at any value: calls that may
 * overlap on one GPU (different streams, or threads without ordering) race
 * on it; serialise them, e.g. on one stream. GEMMA3_ERR_HIP also when the
 * array's device address cannot be obtained.
 */
#define GEMMA3_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
int gemma3_attn_decode_static(const gemma3_attn_desc *desc, const void *x,
                              const int32_t *segment_pos, const gemma3_attn_weights *w,
                              void *k_cache, void *v_cache, int32_t S, void *y,
                              void *hip_stream);

/*
 * One Gemma 3 block over the residual stream ("Full Gemma 3 Block", How it
 * works): a = RMSNorm_post_attn(Attn(RMSNorm_pre_attn(x))), h = x + a,
 * m = RMSNorm_post_ffw(FFN(RMSNorm_pre_ffw(h))), y = h + m, where Attn is
 * gemma3_attn_prefill with `attn` and the descriptor, each RMSNorm runs over
 * D with (1 + gamma) and eps = 1e-6, and
 * FFN(u) = (GELU_tanh(u W_g) * (u W_u)) W_d.
 * Weights (device, the descriptor's dtype, 16-byte aligned, caller-owned):
 *   the four norm vectors [D];
 *   w_gating [2, D_ff, D]: W_g rows then W_u rows, output-major (the
 *            module's transposed gating einsum layout);
 *   w_linear [D, D_ff]: output-major, i.e. W_d (D_ff x D) transposed.
 * x and y are [B, T, D] and may not alias. Workspace:
 * gemma3_block_workspace_bytes(desc, D_ff). Errors: those of
 * gemma3_attn_prefill; D_ff < 1 -> GEMMA3_ERR_SHAPE; a NULL weight ->
 * GEMMA3_ERR_NULL; misaligned -> GEMMA3_ERR_ALIGN; bf16 with D_ff not a
 * multiple of 64, or D > 6144 -> GEMMA3_ERR_UNSUPPORTED.
 */
typedef struct {
  gemma3_attn_weights attn;
  const void *pre_attn_norm;
  const void *post_attn_norm;
  const void *pre_ffw_norm;
  const void *post_ffw_norm;
  const void *w_gating;
  const void *w_linear;
} gemma3_block_weights;

size_t gemma3_block_workspace_bytes(const gemma3_attn_desc *desc, int32_t D_ff);
int gemma3_block_prefill(const gemma3_attn_desc *desc, int32_t D_ff, const void *x,
                         const int32_t *segment_pos, const int32_t *kv_valid_len,
                         const gemma3_block_weights *w, void *y, void *workspace,
                         size_t workspace_bytes, void *hip_stream);

/*
 * One decode step of a whole block: x [B, 1, D], one token per row at
 * position segment_pos[b]; the attention sublayer is gemma3_attn_decode on
 * the pre-normed token (so k_cache / v_cache, [B, S, H_kv, d_h], hold the
 * keys and values of this layer's pre-normed stream), the rest as in
 * gemma3_block_prefill. Workspace: gemma3_block_decode_workspace_bytes(desc,
 * D_ff, S). Errors: those of gemma3_attn_decode and gemma3_block_prefill.
 */
size_t gemma3_block_decode_workspace_bytes(const gemma3_attn_desc *desc, int32_t D_ff, int32_t S);
int gemma3_block_decode(const gemma3_attn_desc *desc, int32_t D_ff, const void *x,
                        const int32_t *segment_pos, const gemma3_block_weights *w,
                        void *k_cache, void *v_cache, int32_t S, void *y, void *workspace,
                        size_t workspace_bytes, void *hip_stream);

typedef struct {
  int32_t num_layers;
  int32_t window;          /* W of the local layers */
  float local_theta;       /* 1e4 */
  float local_scale;       /* 1 */
  float global_theta;      /* 1e6 */
  float global_scale;      /* 8 on 4B/12B/27B shapes, 1 otherwise */
} gemma3_stack_config;

/*
 * A routed stack of Gemma 3 blocks ("Global vs Local Layer Routing", How it
 * works; "Full Gemma 3 Block"): layer l is gemma3_block_prefill with type
 * gemma3_layer_attn_type(l, num_layers), that type's (theta, scale) and, on
 * local layers, `window`; each layer's output is the next layer's input, the
 * last layer's is y. The descriptor gives B, T, D, H, H_kv, d_h, query_scale
 * and dtype (its attn_type, window, rope_theta and rope_scale are replaced per
 * layer). `layers` is a host array of num_layers block weights (device
 * tensors as in gemma3_block_prefill). Workspace:
 * gemma3_stack_workspace_bytes(desc, D_ff, cfg). Errors: those of
 * gemma3_block_prefill for any layer, checked for every layer before anything
 * is enqueued; num_layers < 1 -> GEMMA3_ERR_SHAPE; NULL cfg or layers ->
 * GEMMA3_ERR_NULL.
 */
size_t gemma3_stack_workspace_bytes(const gemma3_attn_desc *desc, int32_t D_ff,
                                    const gemma3_stack_config *cfg);
int gemma3_stack_prefill(const gemma3_attn_desc *desc, int32_t D_ff,
                         const gemma3_stack_config *cfg, const void *x,
                         const int32_t *segment_pos, const int32_t *kv_valid_len,
                         const gemma3_block_weights *layers, void *y, void *workspace,
                         size_t workspace_bytes, void *hip_stream);

/*
 * The same routed stack, also filling one left-aligned cache per layer
 * ("Global vs Local Layer Routing", How it works: every layer attends with
 * its own type; "Gemma 3 Attention Block", How it works, Cache): layer l's
 * attention sublayer writes the rotated keys and the values of its own input
 * (the pre-attention-normed stream of layer l, rotated with layer l's theta
 * and scale) into k_caches[l] / v_caches[l] as gemma3_attn_prefill_cache
 * does (valid tokens only, slot = segment_pos, positions outside [0, S)
 * skipped). k_caches and v_caches are HOST arrays of num_layers DEVICE
 * pointers, each cache [B, S, H_kv, d_h] of the descriptor's dtype, 16-byte
 * aligned, caller-owned; they are what gemma3_stack_decode reads. Workspace
 * and y as in gemma3_stack_prefill. Errors: those of gemma3_stack_prefill;
 * NULL arrays or entries -> GEMMA3_ERR_NULL; S < 1 -> GEMMA3_ERR_SHAPE;
 * a misaligned cache -> GEMMA3_ERR_ALIGN; all checked before any enqueue.
 */
int gemma3_stack_prefill_cache(const gemma3_attn_desc *desc, int32_t D_ff,
                               const gemma3_stack_config *cfg, const void *x,
                               const int32_t *segment_pos, const int32_t *kv_valid_len,
                               const gemma3_block_weights *layers, void *const *k_caches,
                               void *const *v_caches, int32_t S, void *y, void *workspace,
                               size_t workspace_bytes, void *hip_stream);

/*
 * One decode step of the routed stack: x [B, 1, D], one token per row at
 * position segment_pos[b]; layer l is gemma3_block_decode with the routed
 * type, that type's (theta, scale) and (local) window, against its own
 * caches k_caches[l] / v_caches[l] (host arrays of device pointers as in
 * gemma3_stack_prefill_cache; each [B, S, H_kv, d_h]); each layer's output
 * is the next one's input, the last one's is y [B, 1, D]. Slot
 * segment_pos[b] of every layer's caches is written. Workspace:
 * gemma3_stack_decode_workspace_bytes(desc, D_ff, cfg, S) (desc.T = 1).
 * Errors: those of gemma3_block_decode for any layer and of
 * gemma3_stack_prefill_cache for the cache arrays, all checked before any
 * enqueue.
 */
size_t gemma3_stack_decode_workspace_bytes(const gemma3_attn_desc *desc, int32_t D_ff,
                                           const gemma3_stack_config *cfg, int32_t S);
int gemma3_stack_decode(const gemma3_attn_desc *desc, int32_t D_ff,
                        const gemma3_stack_config *cfg, const void *x,
                        const int32_t *segment_pos, const gemma3_block_weights *layers,
                        void *const *k_caches, void *const *v_caches, int32_t S, void *y,
                        void *workspace, size_t workspace_bytes, void *hip_stream);

/*
 * Host-only KV-cache footprint of a routed stack ("Gemma 3 Attention Block",
 * Overview: the cache is what grows at long context; "Global vs Local Layer
 * Routing", How it works: local layers only read their last W positions).
 * Per layer K and V of [B, S, H_kv, d_h] elements of `dtype`, the caches the
 * decode entry points of this library read, split by the routed type of each
 * layer (gemma3_layer_attn_type). local_window_bytes is an analytic figure:
 * what the local layers would hold if each kept only min(W, S) slots. No
 * entry point of this library reads a cache of that size (every cache here
 * is indexed by slot = position, so it needs S slots).
 * Errors: NULL out -> GEMMA3_ERR_NULL; a size < 1 -> GEMMA3_ERR_SHAPE;
 * window < 1 -> GEMMA3_ERR_WINDOW; unknown dtype -> GEMMA3_ERR_DTYPE.
 */
typedef struct {
  int32_t n_local, n_global;   /* layers of each type */
  size_t local_bytes;          /* K and V of the local layers, S slots each */
  size_t global_bytes;         /* K and V of the global layers, S slots each */
  size_t local_window_bytes;   /* the local layers at min(W, S) slots each (analytic) */
} gemma3_kv_footprint;

int gemma3_kv_cache_footprint(int32_t num_layers, int32_t B, int32_t S, int32_t H_kv,
                              int32_t d_h, int32_t window, int32_t dtype,
                              gemma3_kv_footprint *out);

/* Total of gemma3_kv_cache_footprint: global_bytes + local_bytes, or with
 * local_window_only != 0 global_bytes + local_window_bytes (the analytic
 * window-only figure). 0 for invalid arguments. */
size_t gemma3_kv_cache_bytes(int32_t num_layers, int32_t B, int32_t S, int32_t H_kv, int32_t d_h,
                             int32_t window, int32_t dtype, int32_t local_window_only);

/* Host-only routing helper ("Global vs Local Layer Routing", How it works):
 * type of layer `layer` in a stack of `num_layers`: P[layer mod 6] with
 * P = (L, L, L, L, L, G). Returns -1 when layer is outside [0, num_layers). */
int gemma3_layer_attn_type(int32_t layer, int32_t num_layers);

/* Static, never-NULL description of a status code. */
const char *gemma3_attn_status_string(int status);

/* GEMMA3_ATTN_ABI_VERSION of the built library. */
int gemma3_attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GEMMA3_ATTN_H */
