// Host-side launchers of the gfx950 kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;

static inline int div_up_h(long a, long b) { return (int)((a + b - 1) / b); }

// The weight operand of every projection is given as two row blocks: rows
// [0, N0) come from B0 and rows [N0, N) from B1 (W_q and W_kv are separate
// caller buffers that together form the [Q|K|V] projection).
// K1: C[M,N] (bf16) = A[M,K] * B[N,K]^T; K % 64 == 0, 16-byte aligned rows.
// Fused epilogue of the bf16 QKV projection: QK-norm, RoPE and alpha on the Q
// and K columns, V written transposed (see launch_gemm_qkv_fused).
struct QkvEpilogue {
  const int32_t *pos;              // [B, T] (flattened rows m = b T + t)
  const bf16 *gamma_q, *gamma_k;   // [d_h]
  bf16 *q, *k, *vt;                // [B,H,T,d_h], [B,Hk,T_pad,d_h], [B,Hk,d_h,T_pad]
  int T, T_pad, H, Hk, d_h;
  float alpha;
  double theta, scale;
};
// y = x [w_q; w_kv]^T with the epilogue above instead of a raw store.
// Requires (H d_h) % 256 == 0 and (H_kv d_h) % 256 == 0.
hipError_t launch_gemm_qkv_fused(const bf16 *x, const bf16 *w_q, const bf16 *w_kv, int N0, int M,
                                 int N, int K, const QkvEpilogue &ep, hipStream_t s);
// The MLP's gate|up projection with the GeGLU activation fused into its
// epilogue: z [M, D_ff] = GELU_tanh(x W_g^T) * (x W_u^T), W_gating [2, D_ff, K]
// (gate rows, then up rows), D_ff a multiple of 128. The gate and up values
// are rounded to bf16 before the activation, as the unfused path stores them.
hipError_t launch_gemm_geglu(const bf16 *x, const bf16 *w_gating, int D_ff, bf16 *z, int M, int K,
                             hipStream_t s);

hipError_t launch_gemm_bf16_nt(const bf16 *A, const bf16 *B0, const bf16 *B1, int N0, bf16 *C,
                               int M, int N, int K, hipStream_t s);
// K1d, whole K per workgroup: Y[M,N] (fp32 or bf16) = A[M,K] * W[N,K]^T; K % 32 == 0.
template <typename OutT>
hipError_t launch_gemv16_bf16_wg(const bf16 *A, const bf16 *W0, const bf16 *W1, int N0, OutT *Y,
                                 int M, int N, int K, hipStream_t s);

// Arguments shared by the norm/RoPE kernels.
struct NormRopeArgs {
  int B, T, H, Hk, d_h, T_pad;
  float theta, scale, alpha;
};

// K2 (prefill): reads raw [B*T, (H+2Hk) d_h] projections; writes q [B,H,T,d_h]
// (normalised, rotated, times alpha), k [B,Hk,T_pad,d_h], vt [B,Hk,d_h,T_pad].
template <typename T>
hipError_t launch_qk_norm_rope(const T *qkv, const int32_t *pos, const T *gamma_q,
                               const T *gamma_k, T *q, T *k, T *vt, const NormRopeArgs &a,
                               hipStream_t s);

// K2d (decode): sums ksplit fp32 partials [ksplit][B][(H+2Hk) d_h]; q -> fp32 [B,H,d_h];
// rotated k and v -> cache slot pos[b] of [B,S,Hk,d_h].
template <typename T>
hipError_t launch_qk_norm_rope_decode(const float *part, int ksplit, const int32_t *pos,
                                      const T *gamma_q, const T *gamma_k, float *q, T *k_cache,
                                      T *v_cache, int S, const NormRopeArgs &a, hipStream_t s);

// K3 (prefill attention, bf16).
// Queries are the T rows of q; their absolute index (the one the causal and
// sliding masks use) is q0 + row. Key s is valid below q0 + kv_len[b]
// (q0 + T without kv_len). A plain prefill has q0 = 0; a chunk after q0
// cached tokens has q0 > 0. Key layouts:
//  * S_cache == 0: k [B, H_kv, T_pad, d_h] and vt [B, H_kv, d_h, T_pad]
//    (the prefill workspace; keys 0 .. T_pad - 1, rows past the valid ones zero);
//  * S_cache > 0: k and vt are the caches themselves, [B, S_cache, H_kv, d_h]
//    each (V key-major as stored); only the valid slots are read, any others
//    may hold anything (NaN included).
struct AttnArgs {
  int B, T, H, Hk, d_h, T_pad;
  int local, window;
  int q0;
  int S_cache;
};
// `partial` (flash_attn_partial_bytes(a) bytes, may be NULL when that is 0)
// holds the split-KV partial outputs. flash_attn_partial_bytes_bound(a) is
// at least that for every q0 (the split plan depends on q0, the bound not).
size_t flash_attn_partial_bytes(const AttnArgs &a);
size_t flash_attn_partial_bytes_bound(const AttnArgs &a);
// gamma_k [d_h] bounds the key norms (fixed softmax reference).
// ref_flags (diagnostics, normally 0): kRefExactMax makes every workgroup
// take the exact-row-maximum pass that normally runs only where the logit
// bound is too loose; kRefNoZero keeps every wave off the zero reference.
constexpr int kRefExactMax = 1, kRefNoZero = 2;
hipError_t launch_flash_attn_bf16(const bf16 *q, const bf16 *k, const bf16 *vt,
                                  const int32_t *kv_len, const bf16 *gamma_k, bf16 *o,
                                  void *partial, const AttnArgs &a, int ref_flags,
                                  hipStream_t s);

// K4 + K4c (decode attention): split-KV partials then combine into o [B, H*d_h].
// The partial kernel reads the raw fp32 projections qkv [B, (H + 2 H_kv) d_h]
// and applies QK-norm, RoPE and alpha itself; it also writes the step's
// rotated key and its value into cache slot pos[b].
struct DecodeArgs {
  int B, H, Hk, d_h, S;
  int local, window;
  int chunk, n_chunks;
  float theta, scale, alpha;
};
int decode_chunk(int local, int window, int S, int d_h);
template <typename T>
hipError_t launch_decode_attn(const float *qkv, const T *gamma_q, const T *gamma_k, T *k_cache,
                              T *v_cache, const int32_t *pos, float *part, T *o,
                              const DecodeArgs &a, hipStream_t s);

// Sum of fp32 split partials [ksplit][M][N] into y [M][N].
// Copy the valid tokens' rotated keys (k [B,Hk,T_pad,d_h]) and values
// (vt [B,Hk,d_h,T_pad]) of a prefill into a left-aligned cache [B,S,Hk,d_h]
// at slot pos[b,t].
template <typename T>
hipError_t launch_prefill_cache_write(const T *k, const T *vt, const int32_t *pos,
                                      const int32_t *kv_len, T *k_cache, T *v_cache, int B,
                                      int T_len, int T_pad, int Hk, int d_h, int S,
                                      hipStream_t s);

// Block pieces: out = (res ? res : 0) + RMSNorm(a) (1 + gamma) per row of D
// (D <= 6144), and z = GELU_tanh(g) * u with gu rows [g | u] of 2 D_ff.
template <typename T>
hipError_t launch_rms_norm_add(const T *res, const T *a, const T *gamma, T *out, int M, int D,
                               hipStream_t s);
template <typename T>
hipError_t launch_geglu(const T *gu, T *z, int M, int Dff, hipStream_t s);

template <typename T>
hipError_t launch_splitk_reduce(const float *part, int ksplit, T *y, long MN, hipStream_t s);

// K5: fp32 path (correctness grade).
hipError_t launch_gemm_f32_nt(const float *A, const float *B0, const float *B1, int N0, float *C,
                              int M, int N, int K, hipStream_t s);
hipError_t launch_attn_f32(const float *q, const float *k, const float *vt,
                           const int32_t *kv_len, float *o, const AttnArgs &a, hipStream_t s);
hipError_t launch_gemv_f32(const float *A, const float *W0, const float *W1, int N0, float *P,
                           int M, int N, int K, hipStream_t s);
