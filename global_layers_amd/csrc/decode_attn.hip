// Decode attention against a left-aligned KV cache ("Gemma 3 Attention
// Block", How it works: the step's K and V land in the cache at the query's
// position; the query then attends to cached positions s <= pos, and on local
// layers only to s > pos - W; softmax over those slots mixes V).
//
// HBM-bound split-KV evaluation of that softmax:
//  * The allowed slot range [lo, pos] of row b is cut into chunks of C slots.
//    One workgroup streams one (row, chunk, KV head): K and V rows of that
//    head, d_h contiguous elements per slot, 16-byte loads, each byte read once
//    for all the query heads of the GQA group.
//  * Inside a wave, d_h/32 lanes share one slot (32 channels each); per-slot
//    logits are a short xor-shuffle sum. Each slot group keeps an online
//    softmax state (m, l, acc) per query head; groups and waves are merged by
//    log-sum-exp, and the chunk's (acc, m, l) go to the workspace.
//  * A second kernel merges the chunks of each (row, head) the same way and
//    divides by the total weight. Logits are in log2 units (q pre-scaled by
//    log2 e), so every exponential is an exp2.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace {

constexpr int kDecThreads = 256;
constexpr int kDecUnroll = 4;  // slots per slot group per iteration
constexpr int kChansPerLane = 16;

// Raw 16-channel slice of one cache row held in registers until it is used.
// Lane `sub` of the LPS lanes sharing a slot holds the 16-byte pieces sub,
// sub + LPS, sub + 2 LPS, ... of the row, so each load instruction of the
// slot group covers one contiguous run of 16 LPS bytes (whole cache lines).
// Channel of element i: chan(sub, i).
template <typename T> struct Slice;
template <> struct Slice<bf16> {
  static constexpr int kPer = 8;  // channels per 16-byte piece
  u32x4 v[2];
  template <int LPS> DEVI static int chan(int sub, int i) { return (i / 8) * 8 * LPS + 8 * sub + i % 8; }
  template <int LPS> DEVI void load(const bf16 *row, int sub) {
    v[0] = ld16(row + 8 * sub);
    v[1] = ld16(row + 8 * LPS + 8 * sub);
  }
  DEVI void zero() { v[0] = v[1] = u32x4{0, 0, 0, 0}; }
  DEVI float get(int i) const {
    const bf16x8 h = __builtin_bit_cast(bf16x8, v[i >> 3]);
    return (float)h[i & 7];
  }
};
template <> struct Slice<float> {
  u32x4 v[4];
  template <int LPS> DEVI static int chan(int sub, int i) { return (i / 4) * 4 * LPS + 4 * sub + i % 4; }
  template <int LPS> DEVI void load(const float *row, int sub) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = ld16(row + 4 * LPS * i + 4 * sub);
  }
  DEVI void zero() {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = u32x4{0, 0, 0, 0};
  }
  DEVI float get(int i) const {
    const uint32_t w = v[i >> 2][i & 3];  // scalar copy: bit_cast of a vector element misreads
    return __builtin_bit_cast(float, w);
  }
};

DEVI void row_range(const int32_t *pos, int b, int S, int local, int window, int &lo, int &hi) {
  const int p = pos[b];
  if (p < 0 || p >= S) {
    lo = 0;
    hi = -1;
    return;
  }
  hi = p;
  lo = local ? max(0, p - window + 1) : 0;
}

// grid: x = chunk, y = b, z = kh * n_hgrp + head group. GQ query heads per workgroup.
template <typename T, int D, int GQ>
__global__ void __launch_bounds__(kDecThreads)
decode_attn_partial(const float *__restrict__ q, const T *__restrict__ k_cache,
                    const T *__restrict__ v_cache, const int32_t *__restrict__ pos,
                    float *__restrict__ part, DecodeArgs a, int n_hgrp) {
  constexpr int LPS = D / kChansPerLane;         // lanes per slot
  constexpr int kGroupsPerWave = kWave / LPS;
  constexpr int NG = kGroupsPerWave * (kDecThreads / kWave);
  __shared__ float red[kDecThreads / kWave][GQ][D + 2];

  const int chunk = blockIdx.x, b = blockIdx.y;
  const int kh = blockIdx.z / n_hgrp, hgrp = blockIdx.z % n_hgrp;
  const int G = a.H / a.Hk;
  const int h0 = kh * G + hgrp * GQ;
  int lo, hi;
  row_range(pos, b, a.S, a.local, a.window, lo, hi);
  const int c_lo = lo + chunk * a.chunk;
  if (c_lo > hi) return;  // chunk past this row's range (uniform per block)
  const int c_hi = min(hi, c_lo + a.chunk - 1);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sub = lane % LPS;             // which 16-channel slice
  const int grp = wave * kGroupsPerWave + lane / LPS;

  float qv[GQ][kChansPerLane];
#pragma unroll
  for (int g = 0; g < GQ; ++g) {
    const float *qp = q + ((size_t)b * a.H + h0 + g) * D;
#pragma unroll
    for (int i = 0; i < kChansPerLane; ++i)
      qv[g][i] = qp[Slice<T>::template chan<LPS>(sub, i)] * kLog2e;
  }
  float m[GQ], l[GQ], acc[GQ][kChansPerLane];
#pragma unroll
  for (int g = 0; g < GQ; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int i = 0; i < kChansPerLane; ++i) acc[g][i] = 0.f;
  }

  const size_t slot_stride = (size_t)a.Hk * D;
  const T *kb = k_cache + ((size_t)b * a.S) * slot_stride + (size_t)kh * D;
  const T *vb = v_cache + ((size_t)b * a.S) * slot_stride + (size_t)kh * D;

  for (int s_base = c_lo + grp; s_base <= c_hi; s_base += NG * kDecUnroll) {
    Slice<T> ks[kDecUnroll], vs[kDecUnroll];
    bool ok[kDecUnroll];
    // all K and V loads of the iteration are in flight before any math
#pragma unroll
    for (int u = 0; u < kDecUnroll; ++u) {
      const int s = s_base + u * NG;
      ok[u] = s <= c_hi;
      if (ok[u]) {
        ks[u].template load<LPS>(kb + (size_t)s * slot_stride, sub);
        vs[u].template load<LPS>(vb + (size_t)s * slot_stride, sub);
      } else {
        ks[u].zero();
        vs[u].zero();
      }
    }
    float x[kDecUnroll][GQ];
#pragma unroll
    for (int u = 0; u < kDecUnroll; ++u)
#pragma unroll
      for (int g = 0; g < GQ; ++g) {
        float d = 0.f;
#pragma unroll
        for (int i = 0; i < kChansPerLane; ++i) d = fmaf(qv[g][i], ks[u].get(i), d);
        d = group_sum_dpp<LPS>(d);
        x[u][g] = ok[u] ? d : -INFINITY;
      }
#pragma unroll
    for (int g = 0; g < GQ; ++g) {
      float mx = m[g];
#pragma unroll
      for (int u = 0; u < kDecUnroll; ++u) mx = fmaxf(mx, x[u][g]);
      // slot s_base is valid, so mx is finite
      const float corr = __builtin_amdgcn_exp2f(m[g] - mx);
      m[g] = mx;
      l[g] *= corr;
#pragma unroll
      for (int i = 0; i < kChansPerLane; ++i) acc[g][i] *= corr;
#pragma unroll
      for (int u = 0; u < kDecUnroll; ++u) {
        x[u][g] = __builtin_amdgcn_exp2f(x[u][g] - mx);
        l[g] += x[u][g];
      }
    }
#pragma unroll
    for (int u = 0; u < kDecUnroll; ++u)
#pragma unroll
      for (int g = 0; g < GQ; ++g)
#pragma unroll
        for (int i = 0; i < kChansPerLane; ++i)
          acc[g][i] = fmaf(x[u][g], vs[u].get(i), acc[g][i]);
  }

  // merge the slot groups of this wave (lanes with equal `sub` hold equal channels)
#pragma unroll
  for (int off = LPS; off < kWave; off <<= 1) {
#pragma unroll
    for (int g = 0; g < GQ; ++g) {
      const float mo = __shfl_xor(m[g], off, kWave);
      const float lo_ = __shfl_xor(l[g], off, kWave);
      const float mn = fmaxf(m[g], mo);
      const float mu = mn == -INFINITY ? 0.f : mn;
      const float ea = exp2f(m[g] - mu), eb = exp2f(mo - mu);
      m[g] = mn;
      l[g] = l[g] * ea + lo_ * eb;
#pragma unroll
      for (int i = 0; i < kChansPerLane; ++i) {
        const float ao = __shfl_xor(acc[g][i], off, kWave);
        acc[g][i] = acc[g][i] * ea + ao * eb;
      }
    }
  }
  if (lane < LPS) {
#pragma unroll
    for (int g = 0; g < GQ; ++g) {
#pragma unroll
      for (int i = 0; i < kChansPerLane; ++i)
        red[wave][g][Slice<T>::template chan<LPS>(sub, i)] = acc[g][i];
      if (lane == 0) {
        red[wave][g][D] = m[g];
        red[wave][g][D + 1] = l[g];
      }
    }
  }
  __syncthreads();
  for (int e = tid; e < GQ * D; e += kDecThreads) {
    const int g = e / D, c = e % D;
    float mn = -INFINITY;
#pragma unroll
    for (int wv = 0; wv < kDecThreads / kWave; ++wv) mn = fmaxf(mn, red[wv][g][D]);
    const float mu = mn == -INFINITY ? 0.f : mn;
    float sa = 0.f, sl = 0.f;
#pragma unroll
    for (int wv = 0; wv < kDecThreads / kWave; ++wv) {
      const float wgt = exp2f(red[wv][g][D] - mu);
      sa += wgt * red[wv][g][c];
      sl += wgt * red[wv][g][D + 1];
    }
    float *pp = part + (((size_t)b * a.H + h0 + g) * a.n_chunks + chunk) * (D + 2);
    pp[c] = sa;
    if (c == 0) {
      pp[D] = mn;
      pp[D + 1] = sl;
    }
  }
}

// grid: x = H, y = B; D threads. Each chunk's (m, l) is read once into LDS;
// the chunk weights exp2(m_j - M) are formed there, then each thread sums its
// channel over the chunks with kCombineBatch loads in flight per round trip.
constexpr int kMaxChunks = 128;  // decode_chunk keeps every row at <= 128 chunks
constexpr int kCombineBatch = 32;

template <typename T, int D>
__global__ void __launch_bounds__(D)
decode_attn_combine(const float *__restrict__ part, const int32_t *__restrict__ pos,
                    T *__restrict__ o, DecodeArgs a) {
  __shared__ float m_s[kMaxChunks], l_s[kMaxChunks], wgt[kMaxChunks];
  __shared__ float red[D / 64];
  const int h = blockIdx.x, b = blockIdx.y, c = threadIdx.x;
  const int lane = c & 63, wave = c >> 6;
  int lo, hi;
  row_range(pos, b, a.S, a.local, a.window, lo, hi);
  const int n = hi >= lo ? div_up(hi - lo + 1, a.chunk) : 0;
  const float *pp = part + ((size_t)b * a.H + h) * a.n_chunks * (D + 2);

  float mx = -INFINITY;
  for (int j = c; j < n; j += D) {
    const float2 ml = *reinterpret_cast<const float2 *>(pp + (size_t)j * (D + 2) + D);
    m_s[j] = ml.x;
    l_s[j] = ml.y;
    mx = fmaxf(mx, ml.x);
  }
  mx = wave_max(mx);
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int i = 0; i < D / 64; ++i) M = fmaxf(M, red[i]);
  const float mu = M == -INFINITY ? 0.f : M;
  __syncthreads();
  float sl = 0.f;
  for (int j = c; j < n; j += D) {  // the entries this thread wrote above
    const float wj = exp2f(m_s[j] - mu);
    wgt[j] = wj;
    sl += wj * l_s[j];
  }
  sl = wave_sum(sl);
  if (lane == 0) red[wave] = sl;
  __syncthreads();
  float L = 0.f;
#pragma unroll
  for (int i = 0; i < D / 64; ++i) L += red[i];

  float sa = 0.f;
  for (int j = 0; j < n; j += kCombineBatch) {
    float v[kCombineBatch];
#pragma unroll
    for (int u = 0; u < kCombineBatch; ++u)
      v[u] = j + u < n ? pp[(size_t)(j + u) * (D + 2) + c] : 0.f;
#pragma unroll
    for (int u = 0; u < kCombineBatch; ++u)
      if (j + u < n) sa = fmaf(wgt[j + u], v[u], sa);
  }
  o[((size_t)b * a.H + h) * D + c] = from_f32<T>(L > 0.f ? sa / L : 0.f);
}

template <typename T, int D, int GQ>
hipError_t launch_dec(const float *q, const T *kc, const T *vc, const int32_t *pos, float *part,
                      T *o, const DecodeArgs &a, hipStream_t s) {
  const int G = a.H / a.Hk;
  const int n_hgrp = G / GQ;
  dim3 grid(a.n_chunks, a.B, a.Hk * n_hgrp);
  hipLaunchKernelGGL((decode_attn_partial<T, D, GQ>), grid, dim3(kDecThreads), 0, s, q, kc, vc,
                     pos, part, a, n_hgrp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_attn_combine<T, D>), dim3(a.H, a.B), dim3(D), 0, s, part, pos, o, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_dec_g(const float *q, const T *kc, const T *vc, const int32_t *pos,
                        float *part, T *o, const DecodeArgs &a, hipStream_t s) {
  const int G = a.H / a.Hk;
  if (G % 4 == 0) return launch_dec<T, D, 4>(q, kc, vc, pos, part, o, a, s);
  if (G % 2 == 0) return launch_dec<T, D, 2>(q, kc, vc, pos, part, o, a, s);
  return launch_dec<T, D, 1>(q, kc, vc, pos, part, o, a, s);
}

template <typename T>
__global__ void splitk_reduce(const float *__restrict__ part, int ksplit, T *__restrict__ y,
                              long MN) {
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < MN;
       i += (long)gridDim.x * blockDim.x) {
    float s = 0.f;
    for (int sp = 0; sp < ksplit; ++sp) s += part[(size_t)sp * MN + i];
    y[i] = from_f32<T>(s);
  }
}

}  // namespace

int decode_chunk(int local, int window, int S, int d_h) {
  (void)d_h;
  // local: short chunks so the W slots still spread over many workgroups;
  // global: at most 128 chunks per row, so no workgroup streams for long
  // after the others (a shorter tail) while the combine stays cheap
  const int range = local && window < S ? window : S;
  int c = local ? 64 : 256;  // a workgroup covers 16 slot groups x kDecUnroll slots per pass
  while (div_up_h(range, c) > kMaxChunks) c *= 2;
  return c;
}

template <typename T>
hipError_t launch_decode_attn(const float *q, const T *k_cache, const T *v_cache,
                              const int32_t *pos, float *part, T *o, const DecodeArgs &a,
                              hipStream_t s) {
  switch (a.d_h) {
    case 64: return launch_dec_g<T, 64>(q, k_cache, v_cache, pos, part, o, a, s);
    case 128: return launch_dec_g<T, 128>(q, k_cache, v_cache, pos, part, o, a, s);
    case 256: return launch_dec_g<T, 256>(q, k_cache, v_cache, pos, part, o, a, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
hipError_t launch_splitk_reduce(const float *part, int ksplit, T *y, long MN, hipStream_t s) {
  const int nb = div_up_h(MN, 256);
  const int blocks = nb < 2048 ? nb : 2048;
  hipLaunchKernelGGL(splitk_reduce<T>, dim3(blocks), dim3(256), 0, s, part, ksplit, y, MN);
  return hipGetLastError();
}

template hipError_t launch_decode_attn<bf16>(const float *, const bf16 *, const bf16 *,
                                             const int32_t *, float *, bf16 *,
                                             const DecodeArgs &, hipStream_t);
template hipError_t launch_decode_attn<float>(const float *, const float *, const float *,
                                              const int32_t *, float *, float *,
                                              const DecodeArgs &, hipStream_t);
template hipError_t launch_splitk_reduce<bf16>(const float *, int, bf16 *, long, hipStream_t);
template hipError_t launch_splitk_reduce<float>(const float *, int, float *, long, hipStream_t);
