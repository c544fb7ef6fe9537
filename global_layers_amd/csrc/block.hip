// The residual-stream pieces of a Gemma 3 block ("Full Gemma 3 Block", How it
// works): RMSNorm over D with (1 + gamma) and eps = 1e-6, optionally added to
// a residual (the post-norms sit on the sublayer output, before the add), and
// the GeGLU activation GELU_tanh(g) * u between the MLP's two projections.
// Both are HBM-bound row passes: one workgroup per row for the norm (the row
// stays in registers between the sum of squares and the scaling), a flat
// element-wise pass for the activation. Arithmetic in fp32, one rounding to
// the storage type.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace {

constexpr int kNormThreads = 256;
constexpr int kMaxElems = 24;  // row elements per thread (D <= 256 * 24)
constexpr float kRmsEps = 1e-6f;

template <typename T, int E> struct alignas(sizeof(T) * E) Vec { T e[E]; };

template <typename T, int E>
__global__ void __launch_bounds__(kNormThreads)
rms_norm_add(const T *__restrict__ res, const T *__restrict__ a, const T *__restrict__ gamma,
             T *__restrict__ out, int D) {
  using V = Vec<T, E>;
  const size_t row = blockIdx.x;
  const V *ar = reinterpret_cast<const V *>(a + row * D);
  const int nv = D / E;
  constexpr int kMaxPer = kMaxElems / E;  // vector pieces per thread
  float v[kMaxPer][E];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < kMaxPer; ++i) {
    const int j = threadIdx.x + i * kNormThreads;
    if (j < nv) {
      const V p = ar[j];
#pragma unroll
      for (int k = 0; k < E; ++k) {
        v[i][k] = to_f32(p.e[k]);
        ss = fmaf(v[i][k], v[i][k], ss);
      }
    }
  }
  __shared__ float red[kNormThreads / kWave];
  ss = wave_sum(ss);
  if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < kNormThreads / kWave; ++w) tot += red[w];
  const float inv = rsqrtf(tot / (float)D + kRmsEps);
  const V *gr = reinterpret_cast<const V *>(gamma);
  const V *rr = res ? reinterpret_cast<const V *>(res + row * D) : nullptr;
  V *orow = reinterpret_cast<V *>(out + row * D);
#pragma unroll
  for (int i = 0; i < kMaxPer; ++i) {
    const int j = threadIdx.x + i * kNormThreads;
    if (j < nv) {
      const V g = gr[j];
      V o;
      V r;
      if (rr) r = rr[j];
#pragma unroll
      for (int k = 0; k < E; ++k) {
        float y = v[i][k] * inv * (1.f + to_f32(g.e[k]));
        if (rr) y += to_f32(r.e[k]);
        o.e[k] = from_f32<T>(y);
      }
      orow[j] = o;
    }
  }
}

template <typename T, int E>
__global__ void __launch_bounds__(256)
geglu(const T *__restrict__ gu, T *__restrict__ z, int Dff, long n_vec) {
  using V = Vec<T, E>;
  const int nvr = Dff / E;  // vectors per row of z
  for (long i = blockIdx.x * 256L + threadIdx.x; i < n_vec; i += (long)gridDim.x * 256) {
    const long row = i / nvr;
    const int j = (int)(i % nvr);
    const V g = reinterpret_cast<const V *>(gu + row * 2 * Dff)[j];
    const V u = reinterpret_cast<const V *>(gu + row * 2 * Dff + Dff)[j];
    V o;
#pragma unroll
    for (int k = 0; k < E; ++k) {
      o.e[k] = from_f32<T>(gelu_tanh_times(to_f32(g.e[k]), to_f32(u.e[k])));
    }
    reinterpret_cast<V *>(z + row * Dff)[j] = o;
  }
}

}  // namespace

template <typename T>
hipError_t launch_rms_norm_add(const T *res, const T *a, const T *gamma, T *out, int M, int D,
                               hipStream_t s) {
  if (D > kNormThreads * kMaxElems) return hipErrorInvalidValue;
  if (D % 8 == 0 && sizeof(T) == 2) {
    hipLaunchKernelGGL((rms_norm_add<T, 8>), dim3(M), dim3(kNormThreads), 0, s, res, a, gamma,
                       out, D);
  } else if (D % 4 == 0) {
    hipLaunchKernelGGL((rms_norm_add<T, 4>), dim3(M), dim3(kNormThreads), 0, s, res, a, gamma,
                       out, D);
  } else {
    hipLaunchKernelGGL((rms_norm_add<T, 1>), dim3(M), dim3(kNormThreads), 0, s, res, a, gamma,
                       out, D);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_geglu(const T *gu, T *z, int M, int Dff, hipStream_t s) {
  constexpr int E = 16 / sizeof(T);
  const long n = (long)M * Dff;
  if (Dff % E == 0) {
    const long nv = n / E;
    const unsigned blocks = (unsigned)std::min<long>((nv + 255) / 256, 8192);
    hipLaunchKernelGGL((geglu<T, E>), dim3(blocks), dim3(256), 0, s, gu, z, Dff, nv);
  } else {
    const unsigned blocks = (unsigned)std::min<long>((n + 255) / 256, 8192);
    hipLaunchKernelGGL((geglu<T, 1>), dim3(blocks), dim3(256), 0, s, gu, z, Dff, n);
  }
  return hipGetLastError();
}

template hipError_t launch_rms_norm_add<bf16>(const bf16 *, const bf16 *, const bf16 *, bf16 *,
                                              int, int, hipStream_t);
template hipError_t launch_rms_norm_add<float>(const float *, const float *, const float *,
                                               float *, int, int, hipStream_t);
template hipError_t launch_geglu<bf16>(const bf16 *, bf16 *, int, int, hipStream_t);
template hipError_t launch_geglu<float>(const float *, float *, int, int, hipStream_t);
