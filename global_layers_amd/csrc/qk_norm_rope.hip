// QK-norm, RoPE and the query scale, fused ("QK-Norm", How it works: each
// projected query or key head vector is divided by sqrt(mean(v^2) + 1e-6) and
// multiplied by (1 + gamma), then rotated; "Gemma 3 Attention Block", How it
// works: the query is then scaled by alpha; V is not normalised).
//
// The scalar alpha is folded into the query's (1 + gamma) multiplier: RoPE is
// linear, so scaling before or after the rotation gives the same vector.
//
// RoPE angles: channel pair (i, i + d_h/2) turns by (p / scale) * theta^(-2i/d_h).
// Positions reach 131071, where an fp32 angle would be off by ~1e-2 rad, so
// the angle is formed and reduced modulo 2*pi in fp64; sin/cos run in fp32 on
// the reduced angle.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int kMaxHalf = 128;  // d_h <= 256

// 16-element slices of a head vector: 8 channels of the first half and the
// 8 channels they pair with in the second half (two 16-byte vectors for bf16).
template <typename T> struct Pair8;
template <> struct Pair8<bf16> {
  static DEVI void load(const bf16 *p, int half, float (&a)[8], float (&b)[8]) {
    const bf16x8 u = __builtin_bit_cast(bf16x8, ld16(p));
    const bf16x8 v = __builtin_bit_cast(bf16x8, ld16(p + half));
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = (float)u[i];
      b[i] = (float)v[i];
    }
  }
  static DEVI void store(bf16 *p, int half, const float (&a)[8], const float (&b)[8]) {
    bf16x8 u, v;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      u[i] = (bf16)a[i];
      v[i] = (bf16)b[i];
    }
    st16(p, __builtin_bit_cast(u32x4, u));
    st16(p + half, __builtin_bit_cast(u32x4, v));
  }
};
template <> struct Pair8<float> {
  static DEVI void load(const float *p, int half, float (&a)[8], float (&b)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = p[i];
      b[i] = p[half + i];
    }
  }
  static DEVI void store(float *p, int half, const float (&a)[8], const float (&b)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      p[i] = a[i];
      p[half + i] = b[i];
    }
  }
};

constexpr int kQkUnroll = 2;  // head-vector iterations whose loads are issued together
constexpr int kVtPitch = 64 + 2; // V transpose LDS row pitch (elements), breaks column conflicts

// Q and K heads: one wave per token (4 per block). The token's RoPE (cos, sin)
// are formed once, two pairs per lane, and shared through LDS with every Q
// and K head of the token. A head vector is spread over d_h/16 lanes (8 pairs
// per lane); a wave covers 64/(d_h/16) head vectors per iteration. Key rows
// t in [T, T_pad) are written as zeros.
template <typename T>
DEVI void norm_rope_tokens(const T *__restrict__ qkv, const int32_t *__restrict__ pos,
                           const T *__restrict__ gamma_q, const T *__restrict__ gamma_k,
                           T *__restrict__ q, T *__restrict__ k, const NormRopeArgs &a,
                           int block, char *smem) {
  double *inv_freq = reinterpret_cast<double *>(smem);                       // [kMaxHalf]
  float2 *rot = reinterpret_cast<float2 *>(smem + kMaxHalf * sizeof(double)); // [4][kMaxHalf]
  const int d_h = a.d_h, half = d_h / 2;
  {
    // theta^(-2i/d_h) = 2^(-(2i/d_h) log2 theta), in fp64
    const double l2t = log2((double)a.theta);
    for (int i = threadIdx.x; i < half; i += blockDim.x)
      inv_freq[i] = exp2(-2.0 * (double)i / (double)d_h * l2t);
  }
  __syncthreads();

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const long tok = (long)block * 4 + wave;  // over B * T_pad
  const bool live = tok < (long)a.B * a.T_pad;
  const int b = live ? (int)(tok / a.T_pad) : 0, t = live ? (int)(tok % a.T_pad) : 0;
  float2 *my_rot = rot + wave * kMaxHalf;
  if (live && t < a.T) {
    const int p = pos[(size_t)b * a.T + t];
    const double inv_scale = 1.0 / (double)a.scale;
    for (int i = lane; i < half; i += kWave) {
      float c, sn;
      rope_sincos(p, inv_scale, inv_freq[i], c, sn);
      my_rot[i] = make_float2(c, sn);
    }
  }
  __syncthreads();
  if (!live) return;

  const int lpv = d_h / 16;           // lanes per head vector
  const int vpw = kWave / lpv;        // head vectors per wave iteration
  const int sub = lane % lpv, vec = lane / lpv;
  const int i0 = sub * 8;             // first pair index of this lane
  const int n_heads = a.H + a.Hk;
  const int n_qkv = (a.H + 2 * a.Hk) * d_h;

  if (t >= a.T) {  // padding row: zero keys
    for (int j = vec; j < a.Hk; j += vpw) {
      const float z[8] = {};
      Pair8<T>::store(k + (((size_t)b * a.Hk + j) * a.T_pad + t) * d_h + i0, half, z, z);
    }
    return;
  }

  float cs[8], sn[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float2 r = my_rot[i0 + i];
    cs[i] = r.x;
    sn[i] = r.y;
  }
  float gq1[8], gq2[8], gk1[8], gk2[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    gq1[i] = (1.f + to_f32(gamma_q[i0 + i])) * a.alpha;
    gq2[i] = (1.f + to_f32(gamma_q[half + i0 + i])) * a.alpha;
    gk1[i] = 1.f + to_f32(gamma_k[i0 + i]);
    gk2[i] = 1.f + to_f32(gamma_k[half + i0 + i]);
  }

  const T *src = qkv + ((size_t)b * a.T + t) * n_qkv + i0;
  const int n_iter = div_up(n_heads, vpw);
  for (int it0 = 0; it0 < n_iter; it0 += kQkUnroll) {
    float x1[kQkUnroll][8], x2[kQkUnroll][8];
#pragma unroll
    for (int u = 0; u < kQkUnroll; ++u) {
      const int j = (it0 + u) * vpw + vec;
      if (j < n_heads) {
        Pair8<T>::load(src + (size_t)j * d_h, half, x1[u], x2[u]);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) x1[u][i] = x2[u][i] = 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < kQkUnroll; ++u) {
      const int j = (it0 + u) * vpw + vec;
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) ss += x1[u][i] * x1[u][i] + x2[u][i] * x2[u][i];
      // sum over the lpv lanes of this head vector (aligned lane groups)
      for (int o = lpv / 2; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, kWave);
      if (j >= n_heads) continue;
      const float r = rsqrtf(ss / (float)d_h + 1e-6f);
      const bool is_q = j < a.H;
      float o1[8], o2[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float y1 = x1[u][i] * r * (is_q ? gq1[i] : gk1[i]);
        const float y2 = x2[u][i] * r * (is_q ? gq2[i] : gk2[i]);
        o1[i] = y1 * cs[i] - y2 * sn[i];
        o2[i] = y2 * cs[i] + y1 * sn[i];
      }
      T *dst = is_q ? q + (((size_t)b * a.H + j) * a.T + t) * d_h + i0
                    : k + (((size_t)b * a.Hk + (j - a.H)) * a.T_pad + t) * d_h + i0;
      Pair8<T>::store(dst, half, o1, o2);
    }
  }
}

// V heads: tiles of 64 tokens x 64 channels -> vt[b][kh][c][t0 .. t0+63]
// through LDS, 16-byte global loads and stores (bf16) on both sides.
// Tile index: ((b * Hk + kh) * ceil(d_h / 64) + channel tile) * (T_pad / 64) + token tile.
template <typename T>
DEVI void v_transpose_tile(const T *__restrict__ qkv, T *__restrict__ vt, const NormRopeArgs &a,
                           int tile_id, char *smem) {
  constexpr int kE = 16 / sizeof(T);  // elements per 16-byte vector
  T (*tile)[kVtPitch] = reinterpret_cast<T (*)[kVtPitch]>(smem);
  const int n_tt = a.T_pad / 64, n_ct = div_up(a.d_h, 64);
  const int t0 = (tile_id % n_tt) * 64, c0 = ((tile_id / n_tt) % n_ct) * 64;
  const int bk = tile_id / (n_tt * n_ct);
  const int b = bk / a.Hk, kh = bk % a.Hk, d_h = a.d_h;
  const int n_qkv = (a.H + 2 * a.Hk) * d_h;
  const int j = a.H + a.Hk + kh;
  constexpr int kVecPerRow = 64 / kE;
  for (int e = threadIdx.x; e < 64 * kVecPerRow; e += 256) {
    const int tt = e / kVecPerRow, cv = (e % kVecPerRow) * kE, t = t0 + tt;
    if (c0 + cv >= d_h) continue;  // d_h < 64 (fp32 path)
    T v[kE];
    if (t < a.T) {
      const u32x4 raw = ld16(qkv + ((size_t)b * a.T + t) * n_qkv + j * d_h + c0 + cv);
      const T *rv = reinterpret_cast<const T *>(&raw);
#pragma unroll
      for (int i = 0; i < kE; ++i) v[i] = rv[i];
    } else {
#pragma unroll
      for (int i = 0; i < kE; ++i) v[i] = from_f32<T>(0.f);
    }
#pragma unroll
    for (int i = 0; i < kE; ++i) tile[tt][cv + i] = v[i];
  }
  __syncthreads();
  T *dst = vt + (((size_t)b * a.Hk + kh) * d_h + c0) * a.T_pad + t0;
  for (int e = threadIdx.x; e < 64 * kVecPerRow; e += 256) {
    const int c = e / kVecPerRow, tv = (e % kVecPerRow) * kE;
    if (c0 + c >= d_h) continue;
    T v[kE];
#pragma unroll
    for (int i = 0; i < kE; ++i) v[i] = tile[tv + i][c];
    st16(dst + (size_t)c * a.T_pad + tv, *reinterpret_cast<const u32x4 *>(v));
  }
}

template <typename T> constexpr int norm_smem_bytes() {
  constexpr int rope = kMaxHalf * sizeof(double) + 4 * kMaxHalf * sizeof(float2);
  constexpr int vt = 64 * kVtPitch * sizeof(T);
  return rope > vt ? rope : vt;
}

// One launch for the whole stage: blocks [0, n_tok_blocks) run the Q/K heads
// of 4 tokens each, the rest transpose one V tile each, so the two memory
// passes overlap instead of running back to back.
template <typename T>
__global__ void __launch_bounds__(256)
qk_norm_rope_prefill(const T *__restrict__ qkv, const int32_t *__restrict__ pos,
                     const T *__restrict__ gamma_q, const T *__restrict__ gamma_k,
                     T *__restrict__ q, T *__restrict__ k, T *__restrict__ vt, NormRopeArgs a,
                     int n_tok_blocks) {
  __shared__ __attribute__((aligned(16))) char smem[norm_smem_bytes<T>()];
  if ((int)blockIdx.x < n_tok_blocks)
    norm_rope_tokens<T>(qkv, pos, gamma_q, gamma_k, q, k, a, blockIdx.x, smem);
  else
    v_transpose_tile<T>(qkv, vt, a, blockIdx.x - n_tok_blocks, smem);
}

// grid: x = B, y = H + 2 Hk; one wave per (row, head vector).
template <typename T>
__global__ void __launch_bounds__(64)
qk_norm_rope_decode(const float *__restrict__ part, int ksplit, const int32_t *__restrict__ pos,
                    const T *__restrict__ gamma_q, const T *__restrict__ gamma_k,
                    float *__restrict__ q, T *__restrict__ k_cache, T *__restrict__ v_cache,
                    int S, NormRopeArgs a) {
  const int b = blockIdx.x, j = blockIdx.y, lane = threadIdx.x;
  const int d_h = a.d_h, half = d_h / 2;
  const int n_qkv = (a.H + 2 * a.Hk) * d_h;
  const int p = pos[b];
  const bool slot_ok = p >= 0 && p < S;
  constexpr int kMaxPairs = kMaxHalf / 64;

  float x1[kMaxPairs], x2[kMaxPairs];
  float ss = 0.f;
#pragma unroll
  for (int u = 0; u < kMaxPairs; ++u) {
    const int i = lane + 64 * u;
    float s1 = 0.f, s2 = 0.f;
    if (i < half) {
      for (int sp = 0; sp < ksplit; ++sp) {
        const float *src = part + ((size_t)sp * a.B + b) * n_qkv + j * d_h;
        s1 += src[i];
        s2 += src[i + half];
      }
    }
    x1[u] = s1;
    x2[u] = s2;
    ss += s1 * s1 + s2 * s2;
  }

  if (j >= a.H + a.Hk) {  // V: straight into the cache slot
    if (!slot_ok) return;
    T *dst = v_cache + (((size_t)b * S + p) * a.Hk + (j - a.H - a.Hk)) * d_h;
#pragma unroll
    for (int u = 0; u < kMaxPairs; ++u) {
      const int i = lane + 64 * u;
      if (i < half) {
        dst[i] = from_f32<T>(x1[u]);
        dst[i + half] = from_f32<T>(x2[u]);
      }
    }
    return;
  }

  const bool is_q = j < a.H;
  const T *gamma = is_q ? gamma_q : gamma_k;
  const float mul = is_q ? a.alpha : 1.0f;
  ss = wave_sum(ss);
  const float r = rsqrtf(ss / (float)d_h + 1e-6f);
  const double inv_scale = 1.0 / (double)a.scale;
  // theta^(-2i/d_h) = 2^(-(2i/d_h) log2 theta), in fp64 (as in the prefill kernel)
  const double l2t = log2((double)a.theta);
#pragma unroll
  for (int u = 0; u < kMaxPairs; ++u) {
    const int i = lane + 64 * u;
    if (i >= half) continue;
    const double inv_freq = exp2(-2.0 * (double)i / (double)d_h * l2t);
    float c, s;
    rope_sincos(p, inv_scale, inv_freq, c, s);
    const float y1 = x1[u] * r * (1.f + to_f32(gamma[i])) * mul;
    const float y2 = x2[u] * r * (1.f + to_f32(gamma[i + half])) * mul;
    const float o1 = y1 * c - y2 * s, o2 = y2 * c + y1 * s;
    if (is_q) {
      float *dst = q + ((size_t)b * a.H + j) * d_h;
      dst[i] = o1;
      dst[i + half] = o2;
    } else if (slot_ok) {
      T *dst = k_cache + (((size_t)b * S + p) * a.Hk + (j - a.H)) * d_h;
      dst[i] = from_f32<T>(o1);
      dst[i + half] = from_f32<T>(o2);
    }
  }
}

}  // namespace

template <typename T>
hipError_t launch_qk_norm_rope(const T *qkv, const int32_t *pos, const T *gamma_q,
                               const T *gamma_k, T *q, T *k, T *vt, const NormRopeArgs &a,
                               hipStream_t s) {
  const long toks = (long)a.B * a.T_pad;
  const int n_tok_blocks = (int)div_up_h(toks, 4);
  const long n_vt = (long)(a.T_pad / 64) * div_up_h(a.d_h, 64) * a.B * a.Hk;
  hipLaunchKernelGGL(qk_norm_rope_prefill<T>, dim3((unsigned)(n_tok_blocks + n_vt)), dim3(256), 0,
                     s, qkv, pos, gamma_q, gamma_k, q, k, vt, a, n_tok_blocks);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_qk_norm_rope_decode(const float *part, int ksplit, const int32_t *pos,
                                      const T *gamma_q, const T *gamma_k, float *q, T *k_cache,
                                      T *v_cache, int S, const NormRopeArgs &a, hipStream_t s) {
  dim3 grid(a.B, a.H + 2 * a.Hk);
  hipLaunchKernelGGL(qk_norm_rope_decode<T>, grid, dim3(64), 0, s, part, ksplit, pos, gamma_q,
                     gamma_k, q, k_cache, v_cache, S, a);
  return hipGetLastError();
}

template hipError_t launch_qk_norm_rope<float>(const float *, const int32_t *, const float *,
                                               const float *, float *, float *, float *,
                                               const NormRopeArgs &, hipStream_t);
template hipError_t launch_qk_norm_rope<bf16>(const bf16 *, const int32_t *, const bf16 *,
                                              const bf16 *, bf16 *, bf16 *, bf16 *,
                                              const NormRopeArgs &, hipStream_t);
template hipError_t launch_qk_norm_rope_decode<float>(const float *, int, const int32_t *,
                                                      const float *, const float *, float *,
                                                      float *, float *, int,
                                                      const NormRopeArgs &, hipStream_t);
template hipError_t launch_qk_norm_rope_decode<bf16>(const float *, int, const int32_t *,
                                                     const bf16 *, const bf16 *, float *, bf16 *,
                                                     bf16 *, int, const NormRopeArgs &,
                                                     hipStream_t);
