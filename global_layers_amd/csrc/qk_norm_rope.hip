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

constexpr int kTokBlock = 64;  // tokens per workgroup (one V transpose tile)
constexpr int kMaxHalf = 128;  // d_h <= 256
constexpr int kTileC = 128;    // channels per transpose pass

DEVI void rope_sincos(int p, double inv_scale, double inv_freq, float &c, float &s) {
  const double two_pi = 6.283185307179586476925286766559;
  double a = (double)p * inv_scale * inv_freq;
  a -= rint(a * (1.0 / two_pi)) * two_pi;
  sincosf((float)a, &s, &c);
}

// grid: x = B * (T_pad / 64) token blocks, y = H + 2 Hk head vectors; 256 threads.
template <typename T>
__global__ void __launch_bounds__(256)
qk_norm_rope_prefill(const T *__restrict__ qkv, const int32_t *__restrict__ pos,
                     const T *__restrict__ gamma_q, const T *__restrict__ gamma_k,
                     T *__restrict__ q, T *__restrict__ k, T *__restrict__ vt, NormRopeArgs a) {
  __shared__ double inv_freq[kMaxHalf];
  __shared__ T tile[kTokBlock][kTileC + 1];  // V transpose tile (odd row pitch)

  const int blocks_per_row = a.T_pad / kTokBlock;
  const int b = blockIdx.x / blocks_per_row;
  const int t0 = (blockIdx.x % blocks_per_row) * kTokBlock;
  const int j = blockIdx.y;
  const int d_h = a.d_h, half = d_h / 2;
  const int n_qkv = (a.H + 2 * a.Hk) * d_h;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

  if (j >= a.H + a.Hk) {
    // V head: transpose [64 tokens][d_h] -> vt[b][kh][c][t0 .. t0+63], 128 channels at a time
    const int kh = j - a.H - a.Hk;
    T *dst = vt + ((size_t)b * a.Hk + kh) * d_h * a.T_pad + t0;
    for (int c0 = 0; c0 < d_h; c0 += kTileC) {
      const int nc = min(kTileC, d_h - c0);
      for (int e = threadIdx.x; e < kTokBlock * nc; e += blockDim.x) {
        const int tt = e / nc, c = e % nc, t = t0 + tt;
        tile[tt][c] =
            t < a.T ? qkv[((size_t)b * a.T + t) * n_qkv + j * d_h + c0 + c] : from_f32<T>(0.f);
      }
      __syncthreads();
      for (int e = threadIdx.x; e < kTokBlock * nc; e += blockDim.x) {
        const int c = e / kTokBlock, tt = e % kTokBlock;
        dst[(size_t)(c0 + c) * a.T_pad + tt] = tile[tt][c];
      }
      __syncthreads();
    }
    return;
  }

  const bool is_q = j < a.H;
  for (int i = threadIdx.x; i < half; i += blockDim.x)
    inv_freq[i] = pow((double)a.theta, -2.0 * (double)i / (double)d_h);
  __syncthreads();

  const T *gamma = is_q ? gamma_q : gamma_k;
  const float mul = is_q ? a.alpha : 1.0f;
  const double inv_scale = 1.0 / (double)a.scale;
  // each lane owns pairs i = lane + 64 u, u < ceil(half / 64)
  constexpr int kMaxPairs = kMaxHalf / 64;
  float g1[kMaxPairs], g2[kMaxPairs];
#pragma unroll
  for (int u = 0; u < kMaxPairs; ++u) {
    const int i = lane + 64 * u;
    g1[u] = i < half ? (1.f + to_f32(gamma[i])) * mul : 0.f;
    g2[u] = i < half ? (1.f + to_f32(gamma[i + half])) * mul : 0.f;
  }

  for (int tt = wave; tt < kTokBlock; tt += blockDim.x / 64) {
    const int t = t0 + tt;
    T *dst;
    if (is_q) {
      if (t >= a.T) break;
      dst = q + (((size_t)b * a.H + j) * a.T + t) * d_h;
    } else {
      dst = k + (((size_t)b * a.Hk + (j - a.H)) * a.T_pad + t) * d_h;
      if (t >= a.T) {  // zero padding rows of K
        for (int c = lane; c < d_h; c += 64) dst[c] = from_f32<T>(0.f);
        continue;
      }
    }
    const T *src = qkv + ((size_t)b * a.T + t) * n_qkv + j * d_h;
    float x1[kMaxPairs], x2[kMaxPairs];
    float ss = 0.f;
#pragma unroll
    for (int u = 0; u < kMaxPairs; ++u) {
      const int i = lane + 64 * u;
      x1[u] = i < half ? to_f32(src[i]) : 0.f;
      x2[u] = i < half ? to_f32(src[i + half]) : 0.f;
      ss += x1[u] * x1[u] + x2[u] * x2[u];
    }
    ss = wave_sum(ss);
    const float r = rsqrtf(ss / (float)d_h + 1e-6f);
    const int p = pos[(size_t)b * a.T + t];
#pragma unroll
    for (int u = 0; u < kMaxPairs; ++u) {
      const int i = lane + 64 * u;
      if (i >= half) continue;
      float c, s;
      rope_sincos(p, inv_scale, inv_freq[i], c, s);
      const float y1 = x1[u] * r * g1[u], y2 = x2[u] * r * g2[u];
      dst[i] = from_f32<T>(y1 * c - y2 * s);
      dst[i + half] = from_f32<T>(y2 * c + y1 * s);
    }
  }
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
#pragma unroll
  for (int u = 0; u < kMaxPairs; ++u) {
    const int i = lane + 64 * u;
    if (i >= half) continue;
    const double inv_freq = pow((double)a.theta, -2.0 * (double)i / (double)d_h);
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
  dim3 grid(a.B * (a.T_pad / kTokBlock), a.H + 2 * a.Hk);
  hipLaunchKernelGGL(qk_norm_rope_prefill<T>, grid, dim3(256), 0, s, qkv, pos, gamma_q, gamma_k,
                     q, k, vt, a);
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
