// fp32 kernels for the attention block ("Gemma 3 Attention Block", How it
// works), correctness grade: plain fp32 FMA arithmetic, used when the
// descriptor's dtype is fp32. The QK-norm/RoPE and decode kernels are shared
// with the bf16 path through their element-type template.
#include "common.h"
#include "kernels.h"

namespace {

// C[M,N] = A[M,K] * B[N,K]^T, 64x64 tile, 256 threads x (4x4) outputs.
constexpr int kT = 64, kKB = 16;

__global__ void __launch_bounds__(256)
gemm_f32_nt(const float *__restrict__ A, const float *__restrict__ B0,
            const float *__restrict__ B1, int N0, float *__restrict__ C, int M, int N, int K) {
  __shared__ float As[kKB][kT + 4], Bs[kKB][kT + 4];
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  const int m0 = blockIdx.y * kT, n0 = blockIdx.x * kT;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += kKB) {
    for (int e = threadIdx.x; e < kT * kKB; e += 256) {
      const int r = e / kKB, kk = e % kKB;
      const int gm = m0 + r, gn = n0 + r, gk = k0 + kk;
      As[kk][r] = (gm < M && gk < K) ? A[(size_t)gm * K + gk] : 0.f;
      const float *brow = gn < N0 ? B0 + (size_t)gn * K : B1 + (size_t)(gn - N0) * K;
      Bs[kk][r] = (gn < N && gk < K) ? brow[gk] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kKB; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = As[kk][ty * 4 + i];
        b[i] = Bs[kk][tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int gm = m0 + ty * 4 + i;
    if (gm >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int gn = n0 + tx * 4 + j;
      if (gn < N) C[(size_t)gm * N + gn] = acc[i][j];
    }
  }
}

// One wave per (b, h, query row t). Keys are visited 64 at a time (one per
// lane); the softmax state is wave-uniform; o is accumulated d_h/64 channels
// per lane. q [B,H,T,d_h]; k [B,Hk,T_pad,d_h] and vt [B,Hk,d_h,T_pad], or
// with a.S_cache > 0 the caches [B,S_cache,Hk,d_h] themselves. Only allowed
// keys are read.
constexpr int kMaxD = 256;

__global__ void __launch_bounds__(64)
attn_f32(const float *__restrict__ q, const float *__restrict__ k, const float *__restrict__ vt,
         const int32_t *__restrict__ kv_len, float *__restrict__ o, AttnArgs a) {
  __shared__ float qs[kMaxD];
  const int t = blockIdx.x, h = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
  const int D = a.d_h, G = a.H / a.Hk, kh = h / G;
  const int len = a.q0 + (kv_len ? kv_len[b] : a.T);  // keys below it are valid
  for (int c = lane; c < D; c += 64) qs[c] = q[(((size_t)b * a.H + h) * a.T + t) * D + c];
  __syncthreads();

  const int ta = a.q0 + t;  // absolute index of the query
  const int lo = a.local ? max(0, ta - a.window + 1) : 0;
  const int hi = min(ta, len - 1);  // inclusive
  const bool cache = a.S_cache > 0;
  const float *kb = cache ? k + ((size_t)b * a.S_cache * a.Hk + kh) * D
                          : k + ((size_t)b * a.Hk + kh) * a.T_pad * D;
  const float *vb = cache ? vt + ((size_t)b * a.S_cache * a.Hk + kh) * D
                          : vt + ((size_t)b * a.Hk + kh) * D * a.T_pad;
  // element strides: key row of K; key and channel of V
  const size_t ks = cache ? (size_t)a.Hk * D : (size_t)D;
  const size_t vs = cache ? (size_t)a.Hk * D : 1, vc = cache ? 1 : (size_t)a.T_pad;
  float m = -INFINITY, l = 0.f, acc[kMaxD / 64] = {};
  for (int s0 = lo; s0 <= hi; s0 += 64) {
    const int s = s0 + lane;
    float x = -INFINITY;
    if (s <= hi) {
      float d = 0.f;
      for (int c = 0; c < D; ++c) d = fmaf(qs[c], kb[(size_t)s * ks + c], d);
      x = d;
    }
    const float mn = fmaxf(m, wave_max(x));  // finite: key s0 is allowed
    const float corr = expf(m - mn);
    const float p = expf(x - mn);
    l = l * corr + wave_sum(p);
    m = mn;
#pragma unroll
    for (int i = 0; i < kMaxD / 64; ++i) acc[i] *= corr;
    const int n = min(64, hi - s0 + 1);
    for (int j = 0; j < n; ++j) {
      const float pj = __shfl(p, j, kWave);
#pragma unroll
      for (int i = 0; i < kMaxD / 64; ++i) {
        const int c = lane + 64 * i;
        if (c < D) acc[i] = fmaf(pj, vb[(size_t)(s0 + j) * vs + c * vc], acc[i]);
      }
    }
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  float *op = o + ((size_t)b * a.T + t) * ((size_t)a.H * D) + (size_t)h * D;
#pragma unroll
  for (int i = 0; i < kMaxD / 64; ++i) {
    const int c = lane + 64 * i;
    if (c < D) op[c] = acc[i] * inv;
  }
}

// P[0][m][n] = sum_k A[m][k] W[n][k]; one wave per output element (decode sizes).
__global__ void __launch_bounds__(256)
gemv_f32(const float *__restrict__ A, const float *__restrict__ W0, const float *__restrict__ W1,
         int N0, float *__restrict__ P, int M, int N, int K) {
  const int wave = (blockIdx.x * blockDim.x + threadIdx.x) / 64, lane = threadIdx.x & 63;
  if (wave >= M * N) return;
  const int m = wave / N, n = wave % N;
  float s = 0.f;
  const float *w = n < N0 ? W0 + (size_t)n * K : W1 + (size_t)(n - N0) * K;
  for (int kk = lane; kk < K; kk += 64) s = fmaf(A[(size_t)m * K + kk], w[kk], s);
  s = wave_sum(s);
  if (lane == 0) P[(size_t)m * N + n] = s;
}

}  // namespace

hipError_t launch_gemm_f32_nt(const float *A, const float *B0, const float *B1, int N0, float *C,
                              int M, int N, int K, hipStream_t s) {
  hipLaunchKernelGGL(gemm_f32_nt, dim3(div_up_h(N, kT), div_up_h(M, kT)), dim3(256), 0, s, A, B0,
                     B1, N0, C, M, N, K);
  return hipGetLastError();
}

hipError_t launch_attn_f32(const float *q, const float *k, const float *vt,
                           const int32_t *kv_len, float *o, const AttnArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(attn_f32, dim3(a.T, a.H, a.B), dim3(64), 0, s, q, k, vt, kv_len, o, a);
  return hipGetLastError();
}

hipError_t launch_gemv_f32(const float *A, const float *W0, const float *W1, int N0, float *P,
                           int M, int N, int K, hipStream_t s) {
  const long waves = (long)M * N;
  hipLaunchKernelGGL(gemv_f32, dim3(div_up_h(waves, 4)), dim3(256), 0, s, A, W0, W1, N0, P, M, N,
                     K);
  return hipGetLastError();
}
