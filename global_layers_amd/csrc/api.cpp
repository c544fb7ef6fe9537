// C ABI of the attention library: host-side validation, workspace planning
// and the launch sequence of each call ("Gemma 3 Attention Block", How it
// works: projections -> QK-norm -> RoPE -> query scale -> masked grouped
// softmax attention -> output projection; decode adds the cache write).
//
// Every check runs before the first enqueue, so a validation error leaves
// the stream untouched. The library keeps no state between calls.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "../../include/gemma3_attn.h"
#include "../../include/gemma3_attn_stages.h"
#include "kernels.h"

namespace {

constexpr size_t kAlign = 256;
constexpr int kTokPad = 64;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

size_t elem_size(int dtype) { return dtype == GEMMA3_BF16 ? 2 : 4; }

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Shape / scalar validation shared by prefill and decode (S == 0: prefill).
int check_desc(const gemma3_attn_desc *d, int32_t S) {
  if (!d) return GEMMA3_ERR_NULL;
  if (d->B <= 0 || d->T <= 0 || d->D <= 0 || d->H <= 0 || d->H_kv <= 0 || d->d_h <= 0)
    return GEMMA3_ERR_SHAPE;
  if (d->H % d->H_kv != 0 || d->d_h % 2 != 0) return GEMMA3_ERR_SHAPE;
  if (S < 0) return GEMMA3_ERR_SHAPE;
  if (S > 0 && d->T != 1) return GEMMA3_ERR_SHAPE;
  if (d->dtype != GEMMA3_F32 && d->dtype != GEMMA3_BF16) return GEMMA3_ERR_DTYPE;
  if (d->attn_type != GEMMA3_ATTN_GLOBAL && d->attn_type != GEMMA3_ATTN_LOCAL_SLIDING)
    return GEMMA3_ERR_DTYPE;
  if (d->attn_type == GEMMA3_ATTN_LOCAL_SLIDING && d->window < 1) return GEMMA3_ERR_WINDOW;
  if (!isfinite(d->rope_theta) || !isfinite(d->rope_scale) || !isfinite(d->query_scale) ||
      d->rope_theta <= 0.f || d->rope_scale <= 0.f)
    return GEMMA3_ERR_ROPE;
  // int32 index budget of the kernels
  const long n_qkv = (long)(d->H + 2 * d->H_kv) * d->d_h;
  const long widest = n_qkv > d->D ? n_qkv : d->D;
  const long M = (long)d->B * d->T;
  if (M * widest >= (1L << 31) || (long)d->H * d->d_h >= (1L << 31)) return GEMMA3_ERR_UNSUPPORTED;
  if ((long)d->T + kTokPad >= (1L << 31)) return GEMMA3_ERR_UNSUPPORTED;
  if (d->dtype == GEMMA3_BF16) {
    if (d->d_h != 64 && d->d_h != 128 && d->d_h != 256) return GEMMA3_ERR_UNSUPPORTED;
    if (d->D % 64 != 0 || (d->H * d->d_h) % 64 != 0) return GEMMA3_ERR_UNSUPPORTED;
  } else {
    // the norm/RoPE kernel spreads a head over d_h/16 lanes (a power of two)
    if (d->d_h < 16 || d->d_h > 256 || (d->d_h & (d->d_h - 1)) != 0) return GEMMA3_ERR_UNSUPPORTED;
  }
  if (S > 0 && d->d_h % 64 != 0) return GEMMA3_ERR_UNSUPPORTED;  // decode: 32 channels per lane
  return GEMMA3_OK;
}

AttnArgs attn_args(const gemma3_attn_desc *d, int T_pad, int q0 = 0) {
  return AttnArgs{d->B, d->T, d->H, d->H_kv, d->d_h, T_pad,
                  d->attn_type == GEMMA3_ATTN_LOCAL_SLIDING ? 1 : 0, d->window, q0};
}

// Workspace of a prefill chunk: the prefill's (projections, Q, the chunk's
// own K / V^T) followed by room for the attention's split-KV partials (the
// attention reads every key straight from the caches, so nothing here
// depends on how many tokens the caches already hold).
struct ChunkLayout {
  size_t part, total;
};

int layout(const gemma3_attn_desc *d, int32_t S, gemma3_ws_layout *L) {
  int st = check_desc(d, S);
  if (st != GEMMA3_OK) return st;
  memset(L, 0, sizeof(*L));
  const size_t esz = elem_size(d->dtype);
  const size_t n_qkv = (size_t)(d->H + 2 * d->H_kv) * d->d_h;
  size_t off = 0;
  if (S == 0) {
    const size_t M = (size_t)d->B * d->T;
    L->T_pad = div_up_h(d->T, kTokPad) * kTokPad;
    L->qkv = off;
    L->o = off;  // o reuses the raw projection buffer (dead after QK-norm)
    off = align_up(off + M * n_qkv * esz);
    L->q = off;
    off = align_up(off + (size_t)d->B * d->H * d->T * d->d_h * esz);
    L->k = off;
    off = align_up(off + (size_t)d->B * d->H_kv * L->T_pad * d->d_h * esz);
    L->vt = off;
    off = align_up(off + (size_t)d->B * d->H_kv * d->d_h * L->T_pad * esz);
    if (d->dtype == GEMMA3_BF16) {
      const size_t part = flash_attn_partial_bytes(attn_args(d, L->T_pad));
      if (part) {
        L->attn_part = off;
        off = align_up(off + part);
      }
    }
  } else {
    const bool bf = d->dtype == GEMMA3_BF16;
    const bool local = d->attn_type == GEMMA3_ATTN_LOCAL_SLIDING;
    // the bf16 projections run over the whole K per workgroup (no split partials)
    L->ksplit_qkv = 1;
    L->ksplit_out = 1;
    L->chunk = decode_chunk(local, d->window, S, d->d_h);
    const int range = local && d->window < S ? d->window : S;
    L->n_chunks = div_up_h(range, L->chunk);
    L->qkv = off;
    off = align_up(off + (size_t)L->ksplit_qkv * d->B * n_qkv * 4);
    L->q = off;
    off = align_up(off + (size_t)d->B * d->H * d->d_h * 4);
    L->part = off;
    off = align_up(off + (size_t)d->B * d->H * L->n_chunks * (d->d_h + 2) * 4);
    L->o = off;
    off = align_up(off + (size_t)d->B * d->H * d->d_h * esz);
    L->ypart = off;
    off = align_up(off + (size_t)L->ksplit_out * d->B * d->D * 4);
  }
  L->total_bytes = off;
  return GEMMA3_OK;
}

int chunk_layout(const gemma3_attn_desc *d, int32_t start, gemma3_ws_layout *L, ChunkLayout *C) {
  int st = layout(d, 0, L);
  if (st != GEMMA3_OK) return st;
  if (start < 0 || (long)start + d->T > INT32_MAX - kTokPad) return GEMMA3_ERR_SHAPE;
  size_t off = L->total_bytes;
  C->part = off;
  if (d->dtype == GEMMA3_BF16) off = align_up(off + flash_attn_partial_bytes_bound(attn_args(d, L->T_pad)));
  C->total = off;
  return GEMMA3_OK;
}

// Block workspace: the attention's, then the normed stream (pre-attention,
// later pre-MLP), the sublayer output (attention, later MLP), h, the MLP's
// gate|up projection and its activation.
struct BlockLayout {
  size_t hn, a, h, gu, z, total;
};

int block_layout(const gemma3_attn_desc *d, int32_t D_ff, gemma3_ws_layout *L, BlockLayout *K) {
  int st = layout(d, 0, L);
  if (st != GEMMA3_OK) return st;
  if (D_ff < 1) return GEMMA3_ERR_SHAPE;
  if (d->D > 6144) return GEMMA3_ERR_UNSUPPORTED;
  if (d->dtype == GEMMA3_BF16 && D_ff % 64 != 0) return GEMMA3_ERR_UNSUPPORTED;
  const size_t esz = elem_size(d->dtype), M = (size_t)d->B * d->T;
  size_t off = L->total_bytes;
  K->hn = off;
  off = align_up(off + M * d->D * esz);
  K->a = off;
  off = align_up(off + M * d->D * esz);
  K->h = off;
  off = align_up(off + M * d->D * esz);
  K->gu = off;
  off = align_up(off + M * 2 * (size_t)D_ff * esz);
  K->z = off;
  off = align_up(off + M * (size_t)D_ff * esz);
  K->total = off;
  return GEMMA3_OK;
}

// Block decode workspace: the attention decode's, then the normed token, the
// sublayer output, h, gate|up, the activation and (fp32 path) the fp32
// projection outputs before rounding.
struct BlockDecodeLayout {
  size_t hn, a, h, gu, z, part, total;
  int ks_gu, ks_dn;
};

int block_decode_layout(const gemma3_attn_desc *d, int32_t D_ff, int32_t S, gemma3_ws_layout *L,
                        BlockDecodeLayout *K) {
  if (S < 1) return d ? GEMMA3_ERR_SHAPE : GEMMA3_ERR_NULL;
  int st = layout(d, S, L);
  if (st != GEMMA3_OK) return st;
  if (D_ff < 1) return GEMMA3_ERR_SHAPE;
  if (d->D > 6144) return GEMMA3_ERR_UNSUPPORTED;
  const bool bf = d->dtype == GEMMA3_BF16;
  if (bf && D_ff % 64 != 0) return GEMMA3_ERR_UNSUPPORTED;
  const size_t esz = elem_size(d->dtype), B = d->B;
  size_t off = L->total_bytes;
  K->hn = off;
  off = align_up(off + B * d->D * esz);
  K->a = off;
  off = align_up(off + B * d->D * esz);
  K->h = off;
  off = align_up(off + B * d->D * esz);
  K->gu = off;
  off = align_up(off + B * 2 * (size_t)D_ff * esz);
  K->z = off;
  off = align_up(off + B * (size_t)D_ff * esz);
  K->ks_gu = 1;
  K->ks_dn = 1;
  K->part = off;
  const size_t p1 = (size_t)K->ks_gu * B * 2 * D_ff, p2 = (size_t)K->ks_dn * B * d->D;
  off = align_up(off + (p1 > p2 ? p1 : p2) * 4);
  K->total = off;
  return GEMMA3_OK;
}

int check_weights(const gemma3_attn_weights *w) {
  if (!w || !w->w_q || !w->w_kv || !w->w_o || !w->gamma_q || !w->gamma_k) return GEMMA3_ERR_NULL;
  if (!aligned16(w->w_q) || !aligned16(w->w_kv) || !aligned16(w->w_o)) return GEMMA3_ERR_ALIGN;
  return GEMMA3_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? GEMMA3_OK : GEMMA3_ERR_HIP; }

#define RUN(expr)                              \
  do {                                         \
    int _st = hip_status(expr);                \
    if (_st != GEMMA3_OK) return _st;          \
  } while (0)

template <typename T>
int prefill_impl(const gemma3_attn_desc *d, const void *x, const int32_t *pos,
                 const int32_t *kv_len, const gemma3_attn_weights *w, void *y, void *ws,
                 const gemma3_ws_layout &L, hipStream_t s, uint32_t stages) {
  char *base = (char *)ws;
  T *qkv = (T *)(base + L.qkv), *o = (T *)(base + L.o);
  T *q = (T *)(base + L.q), *k = (T *)(base + L.k), *vt = (T *)(base + L.vt);
  const int M = d->B * d->T, Nq = d->H * d->d_h, Nkv = 2 * d->H_kv * d->d_h;
  const bool bf = d->dtype == GEMMA3_BF16;
  // The bf16 attention kernel takes its logits in base-2 units: its queries
  // carry alpha log2(e) (one scale folded in before the single bf16 rounding).
  const float q_scale = bf ? (float)(d->query_scale * 1.4426950408889634) : d->query_scale;

  // Both stages in one kernel when every projection tile holds whole Q, K or
  // V heads: the QK-norm / RoPE / V transpose run in the GEMM's epilogue and
  // the raw projections never reach memory.
  const bool fused = bf && (stages & GEMMA3_STAGE_QKV_PROJ) && (stages & GEMMA3_STAGE_QK_NORM) &&
                     Nq % 256 == 0 && (d->H_kv * d->d_h) % 256 == 0;
  if (fused) {
    QkvEpilogue ep{pos, (const bf16 *)w->gamma_q, (const bf16 *)w->gamma_k,
                   (bf16 *)q, (bf16 *)k, (bf16 *)vt, d->T, L.T_pad, d->H, d->H_kv, d->d_h,
                   q_scale, (double)d->rope_theta, (double)d->rope_scale};
    RUN(launch_gemm_qkv_fused((const bf16 *)x, (const bf16 *)w->w_q, (const bf16 *)w->w_kv, Nq,
                              M, Nq + Nkv, d->D, ep, s));
  }
  if ((stages & GEMMA3_STAGE_QKV_PROJ) && !fused) {
    if (bf)
      RUN(launch_gemm_bf16_nt((const bf16 *)x, (const bf16 *)w->w_q, (const bf16 *)w->w_kv, Nq,
                              (bf16 *)qkv, M, Nq + Nkv, d->D, s));
    else
      RUN(launch_gemm_f32_nt((const float *)x, (const float *)w->w_q, (const float *)w->w_kv, Nq,
                             (float *)qkv, M, Nq + Nkv, d->D, s));
  }
  if ((stages & GEMMA3_STAGE_QK_NORM) && !fused) {
    NormRopeArgs a{d->B, d->T, d->H, d->H_kv, d->d_h, L.T_pad,
                   d->rope_theta, d->rope_scale, q_scale};
    RUN(launch_qk_norm_rope<T>(qkv, pos, (const T *)w->gamma_q, (const T *)w->gamma_k, q, k, vt,
                               a, s));
  }
  if (stages & GEMMA3_STAGE_ATTN) {
    const AttnArgs a = attn_args(d, L.T_pad);
    if (bf)
      RUN(launch_flash_attn_bf16((const bf16 *)q, (const bf16 *)k, (const bf16 *)vt, kv_len,
                                 (const bf16 *)w->gamma_k, (bf16 *)o,
                                 L.attn_part ? base + L.attn_part : nullptr, a,
                                 ((stages & GEMMA3_STAGE_FORCE_EXACT_MAX) ? kRefExactMax : 0) |
                                     ((stages & GEMMA3_STAGE_FORCE_BOUND_REF) ? kRefNoZero : 0),
                                 s));
    else
      RUN(launch_attn_f32((const float *)q, (const float *)k, (const float *)vt, kv_len,
                          (float *)o, a, s));
  }
  if (stages & GEMMA3_STAGE_OUT_PROJ) {
    if (bf)
      RUN(launch_gemm_bf16_nt((const bf16 *)o, (const bf16 *)w->w_o, (const bf16 *)w->w_o, d->D,
                              (bf16 *)y, M, d->D, Nq, s));
    else
      RUN(launch_gemm_f32_nt((const float *)o, (const float *)w->w_o, (const float *)w->w_o, d->D,
                             (float *)y, M, d->D, Nq, s));
  }
  return GEMMA3_OK;
}

template <typename T>
int decode_impl(const gemma3_attn_desc *d, const void *x, const int32_t *pos,
                const gemma3_attn_weights *w, void *kc, void *vc, int32_t S, void *y, void *ws,
                const gemma3_ws_layout &L, hipStream_t s, uint32_t stages) {
  char *base = (char *)ws;
  float *pqkv = (float *)(base + L.qkv), *qf = (float *)(base + L.q);
  float *part = (float *)(base + L.part), *ypart = (float *)(base + L.ypart);
  T *o = (T *)(base + L.o);
  const int B = d->B, Nq = d->H * d->d_h, Nkv = 2 * d->H_kv * d->d_h;
  const bool bf = d->dtype == GEMMA3_BF16;

  if (stages & GEMMA3_DSTAGE_QKV_PROJ) {
    if (bf)
      RUN(launch_gemv16_bf16_wg<float>((const bf16 *)x, (const bf16 *)w->w_q,
                                       (const bf16 *)w->w_kv, Nq, pqkv, B, Nq + Nkv, d->D, s));
    else
      RUN(launch_gemv_f32((const float *)x, (const float *)w->w_q, (const float *)w->w_kv, Nq,
                          pqkv, B, Nq + Nkv, d->D, s));
  }
  // The attention stage forms q (and the step's k, v, written to the cache)
  // itself; the norm stage alone runs the stand-alone kernel (q to the
  // workspace, k and v to the cache) for inspection.
  if ((stages & GEMMA3_DSTAGE_QK_NORM) && !(stages & GEMMA3_DSTAGE_ATTN)) {
    NormRopeArgs a{B, 1, d->H, d->H_kv, d->d_h, 0, d->rope_theta, d->rope_scale, d->query_scale};
    RUN(launch_qk_norm_rope_decode<T>(pqkv, L.ksplit_qkv, pos, (const T *)w->gamma_q,
                                      (const T *)w->gamma_k, qf, (T *)kc, (T *)vc, S, a, s));
  }
  if (stages & GEMMA3_DSTAGE_ATTN) {
    DecodeArgs a{B, d->H, d->H_kv, d->d_h, S,
                 d->attn_type == GEMMA3_ATTN_LOCAL_SLIDING ? 1 : 0, d->window, L.chunk,
                 L.n_chunks, d->rope_theta, d->rope_scale, d->query_scale};
    RUN(launch_decode_attn<T>(pqkv, (const T *)w->gamma_q, (const T *)w->gamma_k, (T *)kc,
                              (T *)vc, pos, part, o, a, s));
  }
  if (stages & GEMMA3_DSTAGE_OUT_PROJ) {
    if (bf) {
      RUN(launch_gemv16_bf16_wg<bf16>((const bf16 *)o, (const bf16 *)w->w_o,
                                      (const bf16 *)w->w_o, d->D, (bf16 *)y, B, d->D, Nq, s));
    } else {
      RUN(launch_gemv_f32((const float *)o, (const float *)w->w_o, (const float *)w->w_o, d->D,
                          ypart, B, d->D, Nq, s));
      RUN(launch_splitk_reduce<T>(ypart, L.ksplit_out, (T *)y, (long)B * d->D, s));
    }
  }
  return GEMMA3_OK;
}

// kc / vc (optional, [B, S, H_kv, d_h]): the attention sublayer also writes
// its rotated keys and values (those of the pre-normed stream) into them, as
// gemma3_attn_prefill_cache does.
template <typename T>
int block_impl(const gemma3_attn_desc *d, int D_ff, const T *x, const int32_t *pos,
               const int32_t *kv_len, const gemma3_block_weights *w, T *y, char *base,
               const gemma3_ws_layout &L, const BlockLayout &K, hipStream_t s,
               T *kc = nullptr, T *vc = nullptr, int32_t S = 0) {
  const int M = d->B * d->T, D = d->D;
  T *hn = (T *)(base + K.hn), *a = (T *)(base + K.a), *h = (T *)(base + K.h);
  T *gu = (T *)(base + K.gu), *z = (T *)(base + K.z);
  RUN(launch_rms_norm_add<T>(nullptr, x, (const T *)w->pre_attn_norm, hn, M, D, s));
  int st = prefill_impl<T>(d, hn, pos, kv_len, &w->attn, a, base, L, s, GEMMA3_STAGE_ALL);
  if (st != GEMMA3_OK) return st;
  if (kc)
    RUN(launch_prefill_cache_write<T>((const T *)(base + L.k), (const T *)(base + L.vt), pos,
                                      kv_len, kc, vc, d->B, d->T, L.T_pad, d->H_kv, d->d_h, S,
                                      s));
  RUN(launch_rms_norm_add<T>(x, a, (const T *)w->post_attn_norm, h, M, D, s));
  RUN(launch_rms_norm_add<T>(nullptr, h, (const T *)w->pre_ffw_norm, hn, M, D, s));
  if constexpr (sizeof(T) == 2) {
    // gate|up projection with the activation in its epilogue (D_ff a multiple
    // of 128), else the projection then the activation pass
    if (D_ff % 128 == 0) {
      RUN(launch_gemm_geglu(hn, (const bf16 *)w->w_gating, D_ff, z, M, D, s));
    } else {
      RUN(launch_gemm_bf16_nt(hn, (const bf16 *)w->w_gating, (const bf16 *)w->w_gating,
                              2 * D_ff, gu, M, 2 * D_ff, D, s));
      RUN(launch_geglu<T>(gu, z, M, D_ff, s));
    }
    RUN(launch_gemm_bf16_nt(z, (const bf16 *)w->w_linear, (const bf16 *)w->w_linear, D, a, M, D,
                            D_ff, s));
  } else {
    RUN(launch_gemm_f32_nt(hn, (const float *)w->w_gating, (const float *)w->w_gating, 2 * D_ff,
                           gu, M, 2 * D_ff, D, s));
    RUN(launch_geglu<T>(gu, z, M, D_ff, s));
    RUN(launch_gemm_f32_nt(z, (const float *)w->w_linear, (const float *)w->w_linear, D, a, M,
                           D, D_ff, s));
  }
  RUN(launch_rms_norm_add<T>(h, a, (const T *)w->post_ffw_norm, y, M, D, s));
  return GEMMA3_OK;
}

template <typename T>
int block_decode_impl(const gemma3_attn_desc *d, int D_ff, const T *x, const int32_t *pos,
                      const gemma3_block_weights *w, void *kc, void *vc, int32_t S, T *y,
                      char *base, const gemma3_ws_layout &L, const BlockDecodeLayout &K,
                      hipStream_t s) {
  const int B = d->B, D = d->D;
  T *hn = (T *)(base + K.hn), *a = (T *)(base + K.a), *h = (T *)(base + K.h);
  T *gu = (T *)(base + K.gu), *z = (T *)(base + K.z);
  float *part = (float *)(base + K.part);
  RUN(launch_rms_norm_add<T>(nullptr, x, (const T *)w->pre_attn_norm, hn, B, D, s));
  int st = decode_impl<T>(d, hn, pos, &w->attn, kc, vc, S, a, base, L, s, GEMMA3_DSTAGE_ALL);
  if (st != GEMMA3_OK) return st;
  RUN(launch_rms_norm_add<T>(x, a, (const T *)w->post_attn_norm, h, B, D, s));
  RUN(launch_rms_norm_add<T>(nullptr, h, (const T *)w->pre_ffw_norm, hn, B, D, s));
  if constexpr (sizeof(T) == 2) {
    RUN(launch_gemv16_bf16_wg<bf16>(hn, (const bf16 *)w->w_gating, (const bf16 *)w->w_gating,
                                    2 * D_ff, gu, B, 2 * D_ff, D, s));
    RUN(launch_geglu<T>(gu, z, B, D_ff, s));
    RUN(launch_gemv16_bf16_wg<bf16>(z, (const bf16 *)w->w_linear, (const bf16 *)w->w_linear, D,
                                    a, B, D, D_ff, s));
  } else {
    RUN(launch_gemv_f32(hn, (const float *)w->w_gating, (const float *)w->w_gating, 2 * D_ff,
                        part, B, 2 * D_ff, D, s));
    RUN(launch_splitk_reduce<T>(part, K.ks_gu, gu, (long)B * 2 * D_ff, s));
    RUN(launch_geglu<T>(gu, z, B, D_ff, s));
    RUN(launch_gemv_f32(z, (const float *)w->w_linear, (const float *)w->w_linear, D, part, B, D,
                        D_ff, s));
    RUN(launch_splitk_reduce<T>(part, K.ks_dn, a, (long)B * D, s));
  }
  RUN(launch_rms_norm_add<T>(h, a, (const T *)w->post_ffw_norm, y, B, D, s));
  return GEMMA3_OK;
}

}  // namespace

extern "C" {

int gemma3_attn_abi_version(void) { return GEMMA3_ATTN_ABI_VERSION; }

const char *gemma3_attn_status_string(int status) {
  switch (status) {
    case GEMMA3_OK: return "ok";
    case GEMMA3_ERR_NULL: return "a required pointer is NULL";
    case GEMMA3_ERR_SHAPE: return "invalid shape (non-positive size, H % H_kv != 0, odd d_h, or T != 1 in decode)";
    case GEMMA3_ERR_WINDOW: return "local layer needs window >= 1";
    case GEMMA3_ERR_DTYPE: return "unknown dtype or attention type";
    case GEMMA3_ERR_ROPE: return "rope_theta and rope_scale must be finite and > 0, query_scale finite";
    case GEMMA3_ERR_WORKSPACE: return "workspace is NULL or smaller than gemma3_attn_workspace_bytes()";
    case GEMMA3_ERR_UNSUPPORTED: return "shape has no kernel in this library";
    case GEMMA3_ERR_HIP: return "a HIP kernel launch failed";
    case GEMMA3_ERR_ALIGN: return "pointer is not 16-byte aligned";
    case GEMMA3_ERR_SCRATCH:
      return "the call needs more workspace than the static scratch holds (GEMMA3_STATIC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int gemma3_layer_attn_type(int32_t layer, int32_t num_layers) {
  if (layer < 0 || layer >= num_layers) return -1;
  // six-slot tile (L, L, L, L, L, G): slot 5 of every tile is global
  return (layer % 6 == 5) ? GEMMA3_ATTN_GLOBAL : GEMMA3_ATTN_LOCAL_SLIDING;
}

int gemma3_attn_workspace_layout(const gemma3_attn_desc *desc, int32_t S, gemma3_ws_layout *out) {
  if (!out) return GEMMA3_ERR_NULL;
  return layout(desc, S, out);
}

size_t gemma3_attn_workspace_bytes(const gemma3_attn_desc *desc, int32_t S) {
  gemma3_ws_layout L;
  return layout(desc, S, &L) == GEMMA3_OK ? L.total_bytes : 0;
}

int gemma3_attn_prefill_stages(const gemma3_attn_desc *desc, const void *x,
                               const int32_t *segment_pos, const int32_t *kv_valid_len,
                               const gemma3_attn_weights *w, void *y, void *workspace,
                               size_t workspace_bytes, void *hip_stream, uint32_t stages) {
  gemma3_ws_layout L;
  int st = layout(desc, 0, &L);
  if (st != GEMMA3_OK) return st;
  if (!x || !segment_pos || !y) return GEMMA3_ERR_NULL;
  if ((st = check_weights(w)) != GEMMA3_OK) return st;
  if (!aligned16(x) || !aligned16(y)) return GEMMA3_ERR_ALIGN;
  if (!workspace || workspace_bytes < L.total_bytes) return GEMMA3_ERR_WORKSPACE;
  if (!aligned16(workspace)) return GEMMA3_ERR_ALIGN;
  hipStream_t s = (hipStream_t)hip_stream;
  if (desc->dtype == GEMMA3_BF16)
    return prefill_impl<bf16>(desc, x, segment_pos, kv_valid_len, w, y, workspace, L, s, stages);
  return prefill_impl<float>(desc, x, segment_pos, kv_valid_len, w, y, workspace, L, s, stages);
}

int gemma3_attn_prefill(const gemma3_attn_desc *desc, const void *x, const int32_t *segment_pos,
                        const int32_t *kv_valid_len, const gemma3_attn_weights *w, void *y,
                        void *workspace, size_t workspace_bytes, void *hip_stream) {
  return gemma3_attn_prefill_stages(desc, x, segment_pos, kv_valid_len, w, y, workspace,
                                    workspace_bytes, hip_stream, GEMMA3_STAGE_ALL);
}

int gemma3_attn_prefill_cache(const gemma3_attn_desc *desc, const void *x,
                              const int32_t *segment_pos, const int32_t *kv_valid_len,
                              const gemma3_attn_weights *w, void *k_cache, void *v_cache,
                              int32_t S, void *y, void *workspace, size_t workspace_bytes,
                              void *hip_stream) {
  if (S < 1) return desc ? GEMMA3_ERR_SHAPE : GEMMA3_ERR_NULL;
  gemma3_ws_layout L;
  int st = layout(desc, 0, &L);
  if (st != GEMMA3_OK) return st;
  if (!k_cache || !v_cache) return GEMMA3_ERR_NULL;
  if (!aligned16(k_cache) || !aligned16(v_cache)) return GEMMA3_ERR_ALIGN;
  if ((long)desc->B * S * desc->H_kv * desc->d_h >= (1L << 62)) return GEMMA3_ERR_UNSUPPORTED;
  // the prefill validates everything else before it enqueues anything
  st = gemma3_attn_prefill_stages(desc, x, segment_pos, kv_valid_len, w, y, workspace,
                                  workspace_bytes, hip_stream, GEMMA3_STAGE_ALL);
  if (st != GEMMA3_OK) return st;
  char *base = (char *)workspace;
  hipStream_t s = (hipStream_t)hip_stream;
  if (desc->dtype == GEMMA3_BF16)
    RUN(launch_prefill_cache_write<bf16>((const bf16 *)(base + L.k), (const bf16 *)(base + L.vt),
                                         segment_pos, kv_valid_len, (bf16 *)k_cache,
                                         (bf16 *)v_cache, desc->B, desc->T, L.T_pad,
                                         desc->H_kv, desc->d_h, S, s));
  else
    RUN(launch_prefill_cache_write<float>((const float *)(base + L.k),
                                          (const float *)(base + L.vt), segment_pos,
                                          kv_valid_len, (float *)k_cache, (float *)v_cache,
                                          desc->B, desc->T, L.T_pad, desc->H_kv, desc->d_h, S,
                                          s));
  return GEMMA3_OK;
}

size_t gemma3_attn_prefill_chunk_workspace_bytes(const gemma3_attn_desc *desc, int32_t start) {
  gemma3_ws_layout L;
  ChunkLayout C;
  return chunk_layout(desc, start, &L, &C) == GEMMA3_OK ? C.total : 0;
}

int gemma3_attn_prefill_chunk(const gemma3_attn_desc *desc, const void *x,
                              const int32_t *segment_pos, const int32_t *kv_valid_len,
                              const gemma3_attn_weights *w, void *k_cache, void *v_cache,
                              int32_t S, int32_t start, void *y, void *workspace,
                              size_t workspace_bytes, void *hip_stream) {
  gemma3_ws_layout L;
  ChunkLayout C;
  int st = chunk_layout(desc, start, &L, &C);
  if (st != GEMMA3_OK) return st;
  if (S < 1 || (long)start + desc->T > S) return GEMMA3_ERR_SHAPE;
  if (!x || !segment_pos || !y || !k_cache || !v_cache) return GEMMA3_ERR_NULL;
  if ((st = check_weights(w)) != GEMMA3_OK) return st;
  if (!aligned16(x) || !aligned16(y) || !aligned16(k_cache) || !aligned16(v_cache))
    return GEMMA3_ERR_ALIGN;
  if ((long)desc->B * S * desc->H_kv * desc->d_h >= (1L << 62)) return GEMMA3_ERR_UNSUPPORTED;
  if (!workspace || workspace_bytes < C.total) return GEMMA3_ERR_WORKSPACE;
  if (!aligned16(workspace)) return GEMMA3_ERR_ALIGN;
  hipStream_t s = (hipStream_t)hip_stream;
  char *base = (char *)workspace;
  // the attention reads every key, the cached ones and the chunk's own, from the caches
  AttnArgs a = attn_args(desc, L.T_pad, start);
  a.S_cache = S;
  // projections with QK-norm / RoPE (Q, and the chunk's K / V^T) ...
  if (desc->dtype == GEMMA3_BF16) {
    st = prefill_impl<bf16>(desc, x, segment_pos, kv_valid_len, w, y, workspace, L, s,
                            GEMMA3_STAGE_QKV_PROJ | GEMMA3_STAGE_QK_NORM);
    if (st != GEMMA3_OK) return st;
    // ... the chunk's keys and values into their slots, attention over the
    // caches, output projection
    RUN(launch_prefill_cache_write<bf16>((const bf16 *)(base + L.k), (const bf16 *)(base + L.vt),
                                         segment_pos, kv_valid_len, (bf16 *)k_cache,
                                         (bf16 *)v_cache, desc->B, desc->T, L.T_pad,
                                         desc->H_kv, desc->d_h, S, s));
    RUN(launch_flash_attn_bf16((const bf16 *)(base + L.q), (const bf16 *)k_cache,
                               (const bf16 *)v_cache, kv_valid_len, (const bf16 *)w->gamma_k,
                               (bf16 *)(base + L.o), C.part < C.total ? base + C.part : nullptr,
                               a, 0, s));
    return prefill_impl<bf16>(desc, x, segment_pos, kv_valid_len, w, y, workspace, L, s,
                              GEMMA3_STAGE_OUT_PROJ);
  }
  st = prefill_impl<float>(desc, x, segment_pos, kv_valid_len, w, y, workspace, L, s,
                           GEMMA3_STAGE_QKV_PROJ | GEMMA3_STAGE_QK_NORM);
  if (st != GEMMA3_OK) return st;
  RUN(launch_prefill_cache_write<float>((const float *)(base + L.k), (const float *)(base + L.vt),
                                        segment_pos, kv_valid_len, (float *)k_cache,
                                        (float *)v_cache, desc->B, desc->T, L.T_pad, desc->H_kv,
                                        desc->d_h, S, s));
  RUN(launch_attn_f32((const float *)(base + L.q), (const float *)k_cache,
                      (const float *)v_cache, kv_valid_len, (float *)(base + L.o), a, s));
  return prefill_impl<float>(desc, x, segment_pos, kv_valid_len, w, y, workspace, L, s,
                             GEMMA3_STAGE_OUT_PROJ);
}

size_t gemma3_block_workspace_bytes(const gemma3_attn_desc *desc, int32_t D_ff) {
  gemma3_ws_layout L;
  BlockLayout K;
  return block_layout(desc, D_ff, &L, &K) == GEMMA3_OK ? K.total : 0;
}


int gemma3_block_prefill(const gemma3_attn_desc *desc, int32_t D_ff, const void *x,
                         const int32_t *segment_pos, const int32_t *kv_valid_len,
                         const gemma3_block_weights *w, void *y, void *workspace,
                         size_t workspace_bytes, void *hip_stream) {
  gemma3_ws_layout L;
  BlockLayout K;
  int st = block_layout(desc, D_ff, &L, &K);
  if (st != GEMMA3_OK) return st;
  if (!x || !segment_pos || !y || !w) return GEMMA3_ERR_NULL;
  if ((st = check_weights(&w->attn)) != GEMMA3_OK) return st;
  const void *bw[6] = {w->pre_attn_norm, w->post_attn_norm, w->pre_ffw_norm, w->post_ffw_norm,
                       w->w_gating, w->w_linear};
  for (const void *p : bw)
    if (!p) return GEMMA3_ERR_NULL;
  for (const void *p : bw)
    if (!aligned16(p)) return GEMMA3_ERR_ALIGN;
  if (!aligned16(x) || !aligned16(y)) return GEMMA3_ERR_ALIGN;
  if (x == y) return GEMMA3_ERR_SHAPE;
  if (!workspace || workspace_bytes < K.total) return GEMMA3_ERR_WORKSPACE;
  if (!aligned16(workspace)) return GEMMA3_ERR_ALIGN;
  hipStream_t s = (hipStream_t)hip_stream;
  if (desc->dtype == GEMMA3_BF16)
    return block_impl<bf16>(desc, D_ff, (const bf16 *)x, segment_pos, kv_valid_len, w, (bf16 *)y,
                            (char *)workspace, L, K, s);
  return block_impl<float>(desc, D_ff, (const float *)x, segment_pos, kv_valid_len, w,
                           (float *)y, (char *)workspace, L, K, s);
}

namespace {
gemma3_attn_desc layer_desc(const gemma3_attn_desc *d, const gemma3_stack_config *c, int l) {
  gemma3_attn_desc e = *d;
  const bool global = gemma3_layer_attn_type(l, c->num_layers) == GEMMA3_ATTN_GLOBAL;
  e.attn_type = global ? GEMMA3_ATTN_GLOBAL : GEMMA3_ATTN_LOCAL_SLIDING;
  e.window = c->window;
  e.rope_theta = global ? c->global_theta : c->local_theta;
  e.rope_scale = global ? c->global_scale : c->local_scale;
  return e;
}

// Every layer's block workspace (the largest), then two residual buffers the
// layers alternate between. S > 0: the decode step's block workspaces, with
// one-token residual buffers.
int stack_layout(const gemma3_attn_desc *d, int32_t D_ff, const gemma3_stack_config *c,
                 int32_t S, size_t *res0, size_t *total) {
  if (!d || !c) return GEMMA3_ERR_NULL;
  if (c->num_layers < 1) return GEMMA3_ERR_SHAPE;
  size_t mx = 0;
  for (int l = 0; l < c->num_layers; ++l) {
    const gemma3_attn_desc e = layer_desc(d, c, l);
    gemma3_ws_layout L;
    size_t tot = 0;
    if (S == 0) {
      BlockLayout K;
      const int st = block_layout(&e, D_ff, &L, &K);
      if (st != GEMMA3_OK) return st;
      tot = K.total;
    } else {
      BlockDecodeLayout K;
      const int st = block_decode_layout(&e, D_ff, S, &L, &K);
      if (st != GEMMA3_OK) return st;
      tot = K.total;
    }
    mx = tot > mx ? tot : mx;
  }
  const size_t res = (size_t)d->B * d->T * d->D * elem_size(d->dtype);
  *res0 = mx;
  *total = align_up(mx + res) + align_up(res);
  return GEMMA3_OK;
}

int check_block_weights(const gemma3_block_weights *w) {
  if (!w) return GEMMA3_ERR_NULL;
  int st = check_weights(&w->attn);
  if (st != GEMMA3_OK) return st;
  const void *bw[6] = {w->pre_attn_norm, w->post_attn_norm, w->pre_ffw_norm, w->post_ffw_norm,
                       w->w_gating, w->w_linear};
  for (const void *p : bw)
    if (!p) return GEMMA3_ERR_NULL;
  for (const void *p : bw)
    if (!aligned16(p)) return GEMMA3_ERR_ALIGN;
  return GEMMA3_OK;
}

// Per-layer caches of a stack: both host arrays present, every entry a
// non-NULL, 16-byte aligned device pointer.
int check_stack_caches(const gemma3_attn_desc *d, int n, void *const *kc, void *const *vc,
                       int32_t S) {
  if (!kc || !vc) return GEMMA3_ERR_NULL;
  if (S < 1) return GEMMA3_ERR_SHAPE;
  for (int l = 0; l < n; ++l) {
    if (!kc[l] || !vc[l]) return GEMMA3_ERR_NULL;
    if (!aligned16(kc[l]) || !aligned16(vc[l])) return GEMMA3_ERR_ALIGN;
  }
  if ((long)d->B * S * d->H_kv * d->d_h >= (1L << 62)) return GEMMA3_ERR_UNSUPPORTED;
  return GEMMA3_OK;
}

// The routed stack of blocks over T tokens (caches optional: kc == NULL).
int stack_prefill_run(const gemma3_attn_desc *desc, int32_t D_ff, const gemma3_stack_config *cfg,
                      const void *x, const int32_t *segment_pos, const int32_t *kv_valid_len,
                      const gemma3_block_weights *layers, void *const *kc, void *const *vc,
                      int32_t S, void *y, void *workspace, size_t workspace_bytes,
                      void *hip_stream) {
  size_t r0, total;
  int st = stack_layout(desc, D_ff, cfg, 0, &r0, &total);
  if (st != GEMMA3_OK) return st;
  if (!x || !segment_pos || !y || !layers) return GEMMA3_ERR_NULL;
  if (!aligned16(x) || !aligned16(y)) return GEMMA3_ERR_ALIGN;
  if (x == y) return GEMMA3_ERR_SHAPE;
  for (int l = 0; l < cfg->num_layers; ++l)
    if ((st = check_block_weights(&layers[l])) != GEMMA3_OK) return st;
  if (kc && (st = check_stack_caches(desc, cfg->num_layers, kc, vc, S)) != GEMMA3_OK) return st;
  if (!workspace || workspace_bytes < total) return GEMMA3_ERR_WORKSPACE;
  if (!aligned16(workspace)) return GEMMA3_ERR_ALIGN;
  char *base = (char *)workspace;
  const size_t res = (size_t)desc->B * desc->T * desc->D * elem_size(desc->dtype);
  void *buf[2] = {base + r0, base + align_up(r0 + res)};
  hipStream_t s = (hipStream_t)hip_stream;
  const void *in = x;
  for (int l = 0; l < cfg->num_layers; ++l) {
    void *out = l == cfg->num_layers - 1 ? y : buf[l & 1];
    const gemma3_attn_desc e = layer_desc(desc, cfg, l);
    gemma3_ws_layout L;
    BlockLayout K;
    if ((st = block_layout(&e, D_ff, &L, &K)) != GEMMA3_OK) return st;
    if (e.dtype == GEMMA3_BF16)
      st = block_impl<bf16>(&e, D_ff, (const bf16 *)in, segment_pos, kv_valid_len, &layers[l],
                            (bf16 *)out, base, L, K, s, kc ? (bf16 *)kc[l] : nullptr,
                            kc ? (bf16 *)vc[l] : nullptr, S);
    else
      st = block_impl<float>(&e, D_ff, (const float *)in, segment_pos, kv_valid_len, &layers[l],
                             (float *)out, base, L, K, s, kc ? (float *)kc[l] : nullptr,
                             kc ? (float *)vc[l] : nullptr, S);
    if (st != GEMMA3_OK) return st;
    in = out;
  }
  return GEMMA3_OK;
}
}  // namespace

size_t gemma3_stack_workspace_bytes(const gemma3_attn_desc *desc, int32_t D_ff,
                                    const gemma3_stack_config *cfg) {
  size_t r0, tot;
  return stack_layout(desc, D_ff, cfg, 0, &r0, &tot) == GEMMA3_OK ? tot : 0;
}

int gemma3_stack_prefill(const gemma3_attn_desc *desc, int32_t D_ff,
                         const gemma3_stack_config *cfg, const void *x,
                         const int32_t *segment_pos, const int32_t *kv_valid_len,
                         const gemma3_block_weights *layers, void *y, void *workspace,
                         size_t workspace_bytes, void *hip_stream) {
  return stack_prefill_run(desc, D_ff, cfg, x, segment_pos, kv_valid_len, layers, nullptr,
                           nullptr, 0, y, workspace, workspace_bytes, hip_stream);
}

int gemma3_stack_prefill_cache(const gemma3_attn_desc *desc, int32_t D_ff,
                               const gemma3_stack_config *cfg, const void *x,
                               const int32_t *segment_pos, const int32_t *kv_valid_len,
                               const gemma3_block_weights *layers, void *const *k_caches,
                               void *const *v_caches, int32_t S, void *y, void *workspace,
                               size_t workspace_bytes, void *hip_stream) {
  if (!k_caches || !v_caches) return GEMMA3_ERR_NULL;
  return stack_prefill_run(desc, D_ff, cfg, x, segment_pos, kv_valid_len, layers, k_caches,
                           v_caches, S, y, workspace, workspace_bytes, hip_stream);
}

size_t gemma3_stack_decode_workspace_bytes(const gemma3_attn_desc *desc, int32_t D_ff,
                                           const gemma3_stack_config *cfg, int32_t S) {
  if (S < 1) return 0;
  size_t r0, tot;
  return stack_layout(desc, D_ff, cfg, S, &r0, &tot) == GEMMA3_OK ? tot : 0;
}

int gemma3_stack_decode(const gemma3_attn_desc *desc, int32_t D_ff,
                        const gemma3_stack_config *cfg, const void *x,
                        const int32_t *segment_pos, const gemma3_block_weights *layers,
                        void *const *k_caches, void *const *v_caches, int32_t S, void *y,
                        void *workspace, size_t workspace_bytes, void *hip_stream) {
  if (S < 1) return desc && cfg ? GEMMA3_ERR_SHAPE : GEMMA3_ERR_NULL;
  size_t r0, total;
  int st = stack_layout(desc, D_ff, cfg, S, &r0, &total);
  if (st != GEMMA3_OK) return st;
  if (!x || !segment_pos || !y || !layers) return GEMMA3_ERR_NULL;
  if (!aligned16(x) || !aligned16(y)) return GEMMA3_ERR_ALIGN;
  if (x == y) return GEMMA3_ERR_SHAPE;
  for (int l = 0; l < cfg->num_layers; ++l)
    if ((st = check_block_weights(&layers[l])) != GEMMA3_OK) return st;
  if ((st = check_stack_caches(desc, cfg->num_layers, k_caches, v_caches, S)) != GEMMA3_OK)
    return st;
  if (!workspace || workspace_bytes < total) return GEMMA3_ERR_WORKSPACE;
  if (!aligned16(workspace)) return GEMMA3_ERR_ALIGN;
  char *base = (char *)workspace;
  const size_t res = (size_t)desc->B * desc->D * elem_size(desc->dtype);
  void *buf[2] = {base + r0, base + align_up(r0 + res)};
  hipStream_t s = (hipStream_t)hip_stream;
  const void *in = x;
  for (int l = 0; l < cfg->num_layers; ++l) {
    void *out = l == cfg->num_layers - 1 ? y : buf[l & 1];
    const gemma3_attn_desc e = layer_desc(desc, cfg, l);
    gemma3_ws_layout L;
    BlockDecodeLayout K;
    if ((st = block_decode_layout(&e, D_ff, S, &L, &K)) != GEMMA3_OK) return st;
    if (e.dtype == GEMMA3_BF16)
      st = block_decode_impl<bf16>(&e, D_ff, (const bf16 *)in, segment_pos, &layers[l],
                                   k_caches[l], v_caches[l], S, (bf16 *)out, base, L, K, s);
    else
      st = block_decode_impl<float>(&e, D_ff, (const float *)in, segment_pos, &layers[l],
                                    k_caches[l], v_caches[l], S, (float *)out, base, L, K, s);
    if (st != GEMMA3_OK) return st;
    in = out;
  }
  return GEMMA3_OK;
}

size_t gemma3_block_decode_workspace_bytes(const gemma3_attn_desc *desc, int32_t D_ff,
                                           int32_t S) {
  gemma3_ws_layout L;
  BlockDecodeLayout K;
  return block_decode_layout(desc, D_ff, S, &L, &K) == GEMMA3_OK ? K.total : 0;
}

int gemma3_block_decode(const gemma3_attn_desc *desc, int32_t D_ff, const void *x,
                        const int32_t *segment_pos, const gemma3_block_weights *w,
                        void *k_cache, void *v_cache, int32_t S, void *y, void *workspace,
                        size_t workspace_bytes, void *hip_stream) {
  gemma3_ws_layout L;
  BlockDecodeLayout K;
  int st = block_decode_layout(desc, D_ff, S, &L, &K);
  if (st != GEMMA3_OK) return st;
  if (!x || !segment_pos || !y || !w || !k_cache || !v_cache) return GEMMA3_ERR_NULL;
  if ((st = check_weights(&w->attn)) != GEMMA3_OK) return st;
  const void *bw[6] = {w->pre_attn_norm, w->post_attn_norm, w->pre_ffw_norm, w->post_ffw_norm,
                       w->w_gating, w->w_linear};
  for (const void *p : bw)
    if (!p) return GEMMA3_ERR_NULL;
  for (const void *p : bw)
    if (!aligned16(p)) return GEMMA3_ERR_ALIGN;
  if (!aligned16(x) || !aligned16(y) || !aligned16(k_cache) || !aligned16(v_cache))
    return GEMMA3_ERR_ALIGN;
  if (x == y) return GEMMA3_ERR_SHAPE;
  if ((long)desc->B * S * desc->H_kv * desc->d_h >= (1L << 62)) return GEMMA3_ERR_UNSUPPORTED;
  if (!workspace || workspace_bytes < K.total) return GEMMA3_ERR_WORKSPACE;
  if (!aligned16(workspace)) return GEMMA3_ERR_ALIGN;
  hipStream_t s = (hipStream_t)hip_stream;
  if (desc->dtype == GEMMA3_BF16)
    return block_decode_impl<bf16>(desc, D_ff, (const bf16 *)x, segment_pos, w, k_cache, v_cache,
                                   S, (bf16 *)y, (char *)workspace, L, K, s);
  return block_decode_impl<float>(desc, D_ff, (const float *)x, segment_pos, w, k_cache, v_cache,
                                  S, (float *)y, (char *)workspace, L, K, s);
}

size_t gemma3_kv_cache_bytes(int32_t num_layers, int32_t B, int32_t S, int32_t H_kv, int32_t d_h,
                             int32_t window, int32_t dtype, int32_t local_window_only) {
  gemma3_kv_footprint f;
  if (gemma3_kv_cache_footprint(num_layers, B, S, H_kv, d_h, window, dtype, &f) != GEMMA3_OK)
    return 0;
  return f.global_bytes + (local_window_only ? f.local_window_bytes : f.local_bytes);
}

int gemma3_kv_cache_footprint(int32_t num_layers, int32_t B, int32_t S, int32_t H_kv,
                              int32_t d_h, int32_t window, int32_t dtype,
                              gemma3_kv_footprint *out) {
  if (!out) return GEMMA3_ERR_NULL;
  memset(out, 0, sizeof(*out));
  if (num_layers < 1 || B < 1 || S < 1 || H_kv < 1 || d_h < 1) return GEMMA3_ERR_SHAPE;
  if (window < 1) return GEMMA3_ERR_WINDOW;
  if (dtype != GEMMA3_F32 && dtype != GEMMA3_BF16) return GEMMA3_ERR_DTYPE;
  const size_t per_slot = 2 * (size_t)B * H_kv * d_h * elem_size(dtype);
  const size_t win = (size_t)(window < S ? window : S);
  for (int l = 0; l < num_layers; ++l) {
    if (gemma3_layer_attn_type(l, num_layers) == GEMMA3_ATTN_LOCAL_SLIDING) {
      ++out->n_local;
      out->local_bytes += per_slot * (size_t)S;
      out->local_window_bytes += per_slot * win;
    } else {
      ++out->n_global;
      out->global_bytes += per_slot * (size_t)S;
    }
  }
  return GEMMA3_OK;
}

int gemma3_attn_decode_stages(const gemma3_attn_desc *desc, const void *x,
                              const int32_t *segment_pos, const gemma3_attn_weights *w,
                              void *k_cache, void *v_cache, int32_t S, void *y, void *workspace,
                              size_t workspace_bytes, void *hip_stream, uint32_t stages) {
  if (S < 1) return desc ? GEMMA3_ERR_SHAPE : GEMMA3_ERR_NULL;
  gemma3_ws_layout L;
  int st = layout(desc, S, &L);
  if (st != GEMMA3_OK) return st;
  if (!x || !segment_pos || !y || !k_cache || !v_cache) return GEMMA3_ERR_NULL;
  if ((st = check_weights(w)) != GEMMA3_OK) return st;
  if (!aligned16(x) || !aligned16(y) || !aligned16(k_cache) || !aligned16(v_cache))
    return GEMMA3_ERR_ALIGN;
  if ((long)desc->B * S * desc->H_kv * desc->d_h >= (1L << 62)) return GEMMA3_ERR_UNSUPPORTED;
  if (!workspace || workspace_bytes < L.total_bytes) return GEMMA3_ERR_WORKSPACE;
  if (!aligned16(workspace)) return GEMMA3_ERR_ALIGN;
  hipStream_t s = (hipStream_t)hip_stream;
  if (desc->dtype == GEMMA3_BF16)
    return decode_impl<bf16>(desc, x, segment_pos, w, k_cache, v_cache, S, y, workspace, L, s,
                             stages);
  return decode_impl<float>(desc, x, segment_pos, w, k_cache, v_cache, S, y, workspace, L, s,
                            stages);
}

int gemma3_attn_decode(const gemma3_attn_desc *desc, const void *x, const int32_t *segment_pos,
                       const gemma3_attn_weights *w, void *k_cache, void *v_cache, int32_t S,
                       void *y, void *workspace, size_t workspace_bytes, void *hip_stream) {
  return gemma3_attn_decode_stages(desc, x, segment_pos, w, k_cache, v_cache, S, y, workspace,
                                   workspace_bytes, hip_stream, GEMMA3_DSTAGE_ALL);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Allocation-free decode: the decode step's workspace lives in a static
// device array, one copy per GPU, resident from the first call on that GPU
// until the process ends. In host code `scratch` is only a stand-in for the
// symbol: the device address of each GPU's copy comes from
// hipGetSymbolAddress, taken once per device with that device current, and
// only that address is ever passed to kernels.
namespace {
static __device__ __align__(256) char scratch[GEMMA3_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch copy (NULL on failure).
void *scratch_of_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}
}  // namespace

extern "C" {

int gemma3_attn_decode_static(const gemma3_attn_desc *desc, const void *x,
                              const int32_t *segment_pos, const gemma3_attn_weights *w,
                              void *k_cache, void *v_cache, int32_t S, void *y,
                              void *hip_stream) {
  if (S < 1) return desc ? GEMMA3_ERR_SHAPE : GEMMA3_ERR_NULL;
  gemma3_ws_layout L;
  int st = layout(desc, S, &L);
  if (st != GEMMA3_OK) return st;
  if (L.total_bytes > GEMMA3_STATIC_SCRATCH_BYTES) return GEMMA3_ERR_SCRATCH;
  void *ws = scratch_of_current_device();
  if (!ws) return GEMMA3_ERR_HIP;
  return gemma3_attn_decode_stages(desc, x, segment_pos, w, k_cache, v_cache, S, y, ws,
                                   GEMMA3_STATIC_SCRATCH_BYTES, hip_stream, GEMMA3_DSTAGE_ALL);
}

}  // extern "C"
