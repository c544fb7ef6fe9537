/*
 * gemma3_attn_stages.h -- stage-level entry points of the attention library.
 *
 * The same work gemma3_attn_prefill / gemma3_attn_decode enqueue, split into
 * its stages so that tests can read the intermediates the workspace holds and
 * a benchmark can time one kernel alone. Arguments, ownership, threading and
 * error behaviour are those of the matching call in gemma3_attn.h; `stages`
 * selects which stages run (in their fixed order). A stage reads what the
 * earlier stages left in the workspace, so running a later stage alone is
 * meaningful only after the earlier ones ran on the same workspace.
 */
#ifndef GEMMA3_ATTN_STAGES_H
#define GEMMA3_ATTN_STAGES_H

#include "gemma3_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Prefill stages ("Gemma 3 Attention Block", How it works). */
#define GEMMA3_STAGE_QKV_PROJ 0x1u  /* [Q|K|V] = x W_q^T | x W_kv^T (q_einsum, kv_einsum)       */
#define GEMMA3_STAGE_QK_NORM 0x2u   /* RMSNorm_Q/K, RoPE, alpha; V transposed ("QK-Norm")      */
#define GEMMA3_STAGE_ATTN 0x4u      /* masked grouped softmax attention -> o                  */
#define GEMMA3_STAGE_OUT_PROJ 0x8u  /* y = o W_o^T (attn_vec_einsum)                          */
#define GEMMA3_STAGE_ALL 0xFu
/* Diagnostic option of the attention stage: every workgroup takes its
 * softmax reference from an exact pass over the row maxima (the path normally
 * used only when the logit bound |q_t| sqrt(d_h) max|1 + gamma_k| is too
 * large for a fixed reference), so tests can check that path on ordinary
 * inputs. Same results up to rounding. */
#define GEMMA3_STAGE_FORCE_EXACT_MAX 0x10u
/* Diagnostic option of the attention stage: no wave takes the zero softmax
 * reference (weights 2^x unshifted, used where every logit bound of the wave
 * is small); the per-row bound is the reference instead, so tests can check
 * that path on ordinary inputs. Same results up to rounding. */
#define GEMMA3_STAGE_FORCE_BOUND_REF 0x20u

/* Decode stages ("Gemma 3 Attention Block", How it works, Cache). */
#define GEMMA3_DSTAGE_QKV_PROJ 0x1u /* raw fp32 projections of the B new tokens              */
#define GEMMA3_DSTAGE_QK_NORM 0x2u  /* alone (without ATTN): norm, RoPE, alpha -> q in the
                                       workspace; k, v into cache slot pos_b                  */
#define GEMMA3_DSTAGE_ATTN 0x4u     /* norm, RoPE, alpha and the cache write inside the
                                       split-KV partial softmax kernel, then the combine     */
#define GEMMA3_DSTAGE_OUT_PROJ 0x8u /* y = o W_o^T                                            */
#define GEMMA3_DSTAGE_ALL 0xFu

/*
 * Byte offsets of the intermediates inside the workspace (all 256-byte
 * aligned). Element type is desc.dtype unless marked fp32.
 * Prefill (S == 0):
 *   qkv  [B*T, (H + 2 H_kv) d_h]  raw projections; reused for o [B*T, H d_h].
 *                                 Not written when QKV_PROJ and QK_NORM run in
 *                                 one call on bf16 with H d_h and H_kv d_h
 *                                 multiples of 256 (one fused kernel then)
 *   q    [B, H, T, d_h]           normalised, rotated, times alpha (bf16: times
 *                                 alpha log2(e), the attention kernel's base-2 logit scale)
 *   k    [B, H_kv, T_pad, d_h]    normalised, rotated (rows T..T_pad-1 zero)
 *   vt   [B, H_kv, d_h, T_pad]    V transposed (columns T..T_pad-1 zero)
 *   attn_part fp32                split-KV partial outputs of the attention stage,
 *                                 [chunks, B, H, T, d_h] then (m, l) per row (only
 *                                 when the grid is too small to fill the GPU)
 *   T_pad = T rounded up to a multiple of 64.
 * Decode (S > 0):
 *   qkv  fp32 [ksplit_qkv, B, (H + 2 H_kv) d_h]  projections (ksplit_qkv is 1)
 *   q    fp32 [B, H, d_h]         normalised, rotated, times alpha (written by the
 *                                 QK_NORM stage when it runs without ATTN)
 *   part fp32 [B, H, n_chunks, d_h + 2]  per-chunk (acc[d_h], m, l), m in log2 units
 *   o    [B, H d_h]               attention output
 *   ypart fp32 [ksplit_out, B, D] output projection before rounding (fp32 path only)
 */
typedef struct {
  size_t total_bytes;
  size_t qkv, q, k, vt, o, part, ypart; /* offsets; unused ones are 0 */
  size_t attn_part;
  int32_t T_pad;                        /* prefill */
  int32_t chunk, n_chunks;              /* decode: cache slots per chunk, chunks per (b, h) */
  int32_t ksplit_qkv, ksplit_out;       /* decode */
} gemma3_ws_layout;

/* Fills *out for desc (S == 0: prefill). Returns a gemma3_status. */
int gemma3_attn_workspace_layout(const gemma3_attn_desc *desc, int32_t S, gemma3_ws_layout *out);

int gemma3_attn_prefill_stages(const gemma3_attn_desc *desc, const void *x,
                               const int32_t *segment_pos, const int32_t *kv_valid_len,
                               const gemma3_attn_weights *w, void *y, void *workspace,
                               size_t workspace_bytes, void *hip_stream, uint32_t stages);

int gemma3_attn_decode_stages(const gemma3_attn_desc *desc, const void *x,
                              const int32_t *segment_pos, const gemma3_attn_weights *w,
                              void *k_cache, void *v_cache, int32_t S, void *y,
                              void *workspace, size_t workspace_bytes, void *hip_stream,
                              uint32_t stages);

#ifdef __cplusplus
}
#endif

#endif /* GEMMA3_ATTN_STAGES_H */
