// Prefill into a left-aligned KV cache ("Gemma 3 Attention Block", How it
// works, Cache: the keys and values of the call are written into a
// left-aligned buffer of S slots, slot = position).
//
// The prefill keeps the rotated keys as k [B, H_kv, T_pad, d_h] and the
// values transposed as vt [B, H_kv, d_h, T_pad]; the cache is
// [B, S, H_kv, d_h]. One workgroup moves a tile of 128 bytes of tokens (64
// bf16 or 32 fp32 tokens, so each V^T row segment is one whole 128-byte line)
// by up to 64 channels of one (row, KV head): K rows are copied as 16-byte
// pieces, V^T is transposed through LDS (16-byte reads along the tokens,
// 16-byte writes along the channels). A token is written when it is valid
// (t < kv_valid_len[b]) and its position lies in [0, S). HBM-bound: each valid
// token moves 2 H_kv d_h elements in and out.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int kCacheThreads = 256;
template <typename T> constexpr int tile_tokens() { return 128 / (int)sizeof(T); }

template <typename T>
__global__ void __launch_bounds__(kCacheThreads)
prefill_cache_write(const T *__restrict__ k, const T *__restrict__ vt,
                    const int32_t *__restrict__ pos, const int32_t *__restrict__ kv_len,
                    T *__restrict__ k_cache, T *__restrict__ v_cache, int T_len, int T_pad,
                    int Hk, int d_h, int S, int cw) {
  constexpr int E = 16 / sizeof(T);  // elements per 16-byte piece
  constexpr int kTT = tile_tokens<T>();
  extern __shared__ __attribute__((aligned(16))) char smem[];
  T *tile = reinterpret_cast<T *>(smem);  // [kTT][cw + E]: a pad piece per token row
  const int pitch = cw + E;
  const int n_cb = d_h / cw;
  const int t0 = blockIdx.x * kTT, kh = blockIdx.y / n_cb, c0 = (blockIdx.y % n_cb) * cw;
  const int b = blockIdx.z;
  const int len = kv_len ? min(kv_len[b], T_len) : T_len;
  const int pc = cw / E;  // pieces per token row segment

  // V^T rows (one channel, kTT tokens) -> tile[token][channel]
  const T *vsrc = vt + (((size_t)b * Hk + kh) * d_h + c0) * T_pad + t0;
  for (int item = threadIdx.x; item < cw * (kTT / E); item += kCacheThreads) {
    const int c = item / (kTT / E), j = item % (kTT / E);
    const u32x4 v = ld16(vsrc + (size_t)c * T_pad + E * j);
    const T *e = reinterpret_cast<const T *>(&v);
#pragma unroll
    for (int i = 0; i < E; ++i) tile[(E * j + i) * pitch + c] = e[i];
  }
  __syncthreads();

  const T *ksrc = k + (((size_t)b * Hk + kh) * T_pad + t0) * d_h + c0;
  for (int item = threadIdx.x; item < kTT * pc; item += kCacheThreads) {
    const int tt = item / pc, j = item % pc;
    const int t = t0 + tt;
    if (t >= len) continue;
    const int p = pos[(size_t)b * T_len + t];
    if (p < 0 || p >= S) continue;
    const size_t dst = (((size_t)b * S + p) * Hk + kh) * d_h + c0 + E * j;
    st16(k_cache + dst, ld16(ksrc + (size_t)tt * d_h + E * j));
    st16(v_cache + dst, ld16(tile + tt * pitch + E * j));
  }
}

}  // namespace

template <typename T>
hipError_t launch_prefill_cache_write(const T *k, const T *vt, const int32_t *pos,
                                      const int32_t *kv_len, T *k_cache, T *v_cache, int B,
                                      int T_len, int T_pad, int Hk, int d_h, int S,
                                      hipStream_t s) {
  constexpr int E = 16 / sizeof(T);
  constexpr int kTT = tile_tokens<T>();
  if (d_h % E != 0 || T_pad % kTT != 0) return hipErrorInvalidValue;
  // channel blocks of up to 64 per workgroup, so that even one short row
  // and one KV head spread over the chip
  const int cw = d_h < 64 ? d_h : 64;
  if (d_h % cw != 0) return hipErrorInvalidValue;
  const size_t lds = (size_t)kTT * (cw + E) * sizeof(T);
  dim3 grid((unsigned)((T_len + kTT - 1) / kTT), (unsigned)(Hk * (d_h / cw)), (unsigned)B);
  hipLaunchKernelGGL(prefill_cache_write<T>, grid, dim3(kCacheThreads), lds, s, k, vt, pos,
                     kv_len, k_cache, v_cache, T_len, T_pad, Hk, d_h, S, cw);
  return hipGetLastError();
}

template hipError_t launch_prefill_cache_write<bf16>(const bf16 *, const bf16 *, const int32_t *,
                                                     const int32_t *, bf16 *, bf16 *, int, int,
                                                     int, int, int, int, hipStream_t);
template hipError_t launch_prefill_cache_write<float>(const float *, const float *,
                                                      const int32_t *, const int32_t *, float *,
                                                      float *, int, int, int, int, int, int,
                                                      hipStream_t);
