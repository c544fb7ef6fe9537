// Prefill attention core on gfx950 MFMA ("Gemma 3 Attention Block", How it
// works: logits = sum_c Q[t,h,c] K[s,h/G,c] with the GQA reshape; causal and
// padding mask, times the sliding mask 1[s > t-W] 1[s < t+W] on local layers;
// blocked logits take the K_MASK fill; softmax over s; weights mix V).
//
// Exact tiled evaluation (online softmax) of that definition:
//  * Blocked logits get exactly zero weight, as K_MASK does in fp32 whenever a
//    row has an allowed key; the fill value itself is never formed. Tiles that
//    no row of the workgroup may see are never visited.
//  * One workgroup = 4 waves = 128 query rows of one KV head: the query heads
//    of a GQA group (up to 4) are packed into the workgroup, so each K/V tile
//    staged in LDS feeds every query head that reads it.
//  * Each wave computes S^T = K Q^T with 32x32x16 bf16 MFMAs: a lane owns one
//    query row and 32 of the 64 keys of a tile, so row max and row sum need
//    one cross-lane step (lane ^ 32). K rows are fed in the permuted order
//    kappa(i) so that the S^T accumulators of a lane are, in register order,
//    the 16-byte B operand of the PV MFMA (O^T += V^T P^T) without moving data.
//  * V arrives transposed ([d_h][T]) so the PV A operand is a contiguous
//    16-byte LDS read.
//  * K and V^T tiles are double-buffered in LDS; the next tile's global loads
//    are issued before the current tile's MFMAs.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int kBN = 64;       // keys per tile
constexpr int kThreads = 256; // 4 waves
constexpr int kRowsPerWave = 32;

template <int D> struct AttnCfg {
  static constexpr int kKPitch = D + 8;       // bf16 elements per K row in LDS
  static constexpr int kVPitch = kBN + 8;     // bf16 elements per V^T row in LDS
  static constexpr int kKElems = kBN * kKPitch;
  static constexpr int kVElems = D * kVPitch;
  static constexpr int kBufElems = kKElems + kVElems;
  static constexpr int kLdsBytes = 2 * kBufElems * 2;
  static constexpr int kKChunks = kBN * D / 8 / kThreads;  // 16-byte chunks per thread
  static constexpr int kVChunks = D * kBN / 8 / kThreads;
  static constexpr int kKS = D / 16;                       // k-steps of the QK^T contraction
  static constexpr int kDB = D / 32;                       // 32-row blocks of O^T
};

// Key permutation inside a 32-key block (see the header comment).
DEVI int kappa(int i) {
  const int g = i >> 3, h = (i >> 2) & 1, r = i & 3;
  return 16 * (g >> 1) + 8 * h + 4 * (g & 1) + r;
}

template <int D>
__global__ void __launch_bounds__(kThreads)
flash_attn_fwd_bf16(const bf16 *__restrict__ q, const bf16 *__restrict__ k,
                    const bf16 *__restrict__ vt, const int32_t *__restrict__ kv_len,
                    bf16 *__restrict__ o, AttnArgs a, int gp, int n_qtiles, int n_hgrp) {
  using Cfg = AttnCfg<D>;
  extern __shared__ __attribute__((aligned(16))) bf16 lds[];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int G = a.H / a.Hk;
  // Logical block order: (b, kh, head group) runs of query tiles, longest
  // (latest) query tile first; runs stay on one XCD.
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int qt = n_qtiles - 1 - bid % n_qtiles;
  int rest = bid / n_qtiles;
  const int hgrp = rest % n_hgrp;
  rest /= n_hgrp;
  const int kh = rest % a.Hk, b = rest / a.Hk;

  const int wpg = 4 / gp;  // waves per query head
  const int hg = w / wpg, tb = w % wpg;
  const int h = kh * G + hgrp * gp + hg;
  const int TQ = kRowsPerWave * wpg;
  const int t_lo = qt * TQ, t_hi = min(a.T, t_lo + TQ);
  const int wq0 = t_lo + tb * kRowsPerWave;       // first query row of this wave
  const int wq_last = min(wq0 + kRowsPerWave, a.T) - 1;
  const int len = kv_len ? kv_len[b] : a.T;

  int kv_begin = a.local ? max(0, t_lo - a.window + 1) : 0;
  const int kv_end = min(t_hi, len);  // exclusive
  const int tile_begin = (kv_begin / kBN) * kBN;

  const int col = lane & 31, hh = lane >> 5;
  const int my_t = wq0 + col;  // this lane's query row

  // Q^T fragments (B operand): query my_t, channels 16 ks + 8 hh + [0, 8).
  bf16x8 qf[Cfg::kKS];
  {
    const bool ok = my_t < a.T;
    const bf16 *qp = q + (((size_t)b * a.H + h) * a.T + (ok ? my_t : 0)) * D + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < Cfg::kKS; ++ks)
      qf[ks] = ok ? *reinterpret_cast<const bf16x8 *>(qp + 16 * ks) : bf16x8{};
  }

  f32x16 acc_o[Cfg::kDB];
#pragma unroll
  for (int i = 0; i < Cfg::kDB; ++i) acc_o[i] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  const bf16 *kbase = k + ((size_t)b * a.Hk + kh) * a.T_pad * D;
  const bf16 *vbase = vt + ((size_t)b * a.Hk + kh) * D * a.T_pad;

  u32x4 rk[Cfg::kKChunks], rv[Cfg::kVChunks];
  auto load_k = [&](int s0) {
#pragma unroll
    for (int i = 0; i < Cfg::kKChunks; ++i) {
      const int c = tid + i * kThreads;
      const int row = c / (D / 8), cc = (c % (D / 8)) * 8;
      rk[i] = ld16(kbase + (size_t)(s0 + row) * D + cc);
    }
  };
  auto load_v = [&](int s0) {
#pragma unroll
    for (int i = 0; i < Cfg::kVChunks; ++i) {
      const int c = tid + i * kThreads;
      const int row = c / (kBN / 8), cc = (c % (kBN / 8)) * 8;
      rv[i] = ld16(vbase + (size_t)row * a.T_pad + s0 + cc);
    }
  };
  auto store_k = [&](int buf) {
    bf16 *ks = lds + buf * Cfg::kBufElems;
#pragma unroll
    for (int i = 0; i < Cfg::kKChunks; ++i) {
      const int c = tid + i * kThreads;
      st16(ks + (c / (D / 8)) * Cfg::kKPitch + (c % (D / 8)) * 8, rk[i]);
    }
  };
  auto store_v = [&](int buf) {
    bf16 *vs = lds + buf * Cfg::kBufElems + Cfg::kKElems;
#pragma unroll
    for (int i = 0; i < Cfg::kVChunks; ++i) {
      const int c = tid + i * kThreads;
      st16(vs + (c / (kBN / 8)) * Cfg::kVPitch + (c % (kBN / 8)) * 8, rv[i]);
    }
  };

  if (kv_end > kv_begin) {
    load_k(tile_begin);
    load_v(tile_begin);
    store_k(0);
    store_v(0);
  }
  __syncthreads();

  const int krow = kappa(col);  // permuted key row this lane feeds
  int buf = 0;
  for (int s0 = tile_begin; s0 < kv_end; s0 += kBN, buf ^= 1) {
    const bool has_next = s0 + kBN < kv_end;
    if (has_next) load_k(s0 + kBN);

    // wave-uniform: does any row of this wave see a key of this tile?
    const bool wave_live = s0 <= wq_last && !(a.local && s0 + kBN - 1 <= wq0 - a.window);
    const bf16 *ks_lds = lds + buf * Cfg::kBufElems;
    const bf16 *vs_lds = ks_lds + Cfg::kKElems;

    f32x16 acc_s[2];
    if (wave_live) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        acc_s[kb] = f32x16{};
        const bf16 *kp = ks_lds + (32 * kb + krow) * Cfg::kKPitch + 8 * hh;
#pragma unroll
        for (int ks = 0; ks < Cfg::kKS; ++ks) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(kp + 16 * ks);
          acc_s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], acc_s[kb], 0, 0, 0);
        }
      }
    }
    if (has_next) {
      store_k(buf ^ 1);
      load_v(s0 + kBN);
    }

    if (wave_live) {
      // tile-uniform mask decision for the whole workgroup
      const bool full = (s0 + kBN - 1 <= t_lo) && (s0 + kBN - 1 < len) &&
                        (!a.local || s0 >= t_hi - a.window);
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          float x = acc_s[kb][e] * kLog2e;
          if (!full) {
            const int g = e >> 2, r = e & 3;
            const int s = s0 + 32 * kb + 16 * (g >> 1) + 8 * hh + 4 * (g & 1) + r;
            const bool ok = s <= my_t && s < len && (!a.local || s > my_t - a.window);
            x = ok ? x : -INFINITY;
          }
          acc_s[kb][e] = x;
          mx = fmaxf(mx, x);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
      const float m_new = fmaxf(m_run, mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float corr = exp2f(m_run - m_use);
      m_run = m_new;
      float psum = 0.f;
      bf16x8 pf[4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = exp2f(acc_s[kb][e] - m_use);
          psum += p;
          pf[2 * kb + (e >> 3)][e & 7] = (bf16)p;
        }
      l_run = l_run * corr + psum;
#pragma unroll
      for (int db = 0; db < Cfg::kDB; ++db) acc_o[db] *= corr;

#pragma unroll
      for (int db = 0; db < Cfg::kDB; ++db) {
        const bf16 *vp = vs_lds + (32 * db + col) * Cfg::kVPitch + 8 * hh;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const bf16x8 vf = *reinterpret_cast<const bf16x8 *>(vp + 16 * kk);
          acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[kk], acc_o[db], 0, 0, 0);
        }
      }
    }
    if (has_next) store_v(buf ^ 1);
    __syncthreads();
  }

  // Normalise and store o[b, t, h, :] (token-major rows of H*d_h).
  const float l_tot = l_run + __shfl_xor(l_run, 32, kWave);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (my_t < a.T) {
    bf16 *op = o + ((size_t)b * a.T + my_t) * ((size_t)a.H * D) + (size_t)h * D;
#pragma unroll
    for (int db = 0; db < Cfg::kDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 v;
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = (bf16)(acc_o[db][4 * g + r] * inv);
        *reinterpret_cast<bf16x4 *>(op + 32 * db + 8 * g + 4 * hh) = v;
      }
  }
}

template <int D>
hipError_t launch_d(const bf16 *q, const bf16 *k, const bf16 *vt, const int32_t *kv_len, bf16 *o,
                    const AttnArgs &a, hipStream_t s) {
  using Cfg = AttnCfg<D>;
  const int G = a.H / a.Hk;
  const int gp = (G % 4 == 0) ? 4 : (G % 2 == 0) ? 2 : 1;
  const int TQ = kRowsPerWave * (4 / gp);
  const int n_qtiles = div_up_h(a.T, TQ);
  const int n_hgrp = G / gp;
  const long n_blocks = (long)a.B * a.Hk * n_hgrp * n_qtiles;
  hipError_t e = hipFuncSetAttribute((const void *)flash_attn_fwd_bf16<D>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     Cfg::kLdsBytes);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(flash_attn_fwd_bf16<D>, dim3((unsigned)n_blocks), dim3(kThreads),
                     Cfg::kLdsBytes, s, q, k, vt, kv_len, o, a, gp, n_qtiles, n_hgrp);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_flash_attn_bf16(const bf16 *q, const bf16 *k, const bf16 *vt,
                                  const int32_t *kv_len, bf16 *o, const AttnArgs &a,
                                  hipStream_t s) {
  switch (a.d_h) {
    case 64: return launch_d<64>(q, k, vt, kv_len, o, a, s);
    case 128: return launch_d<128>(q, k, vt, kv_len, o, a, s);
    case 256: return launch_d<256>(q, k, vt, kv_len, o, a, s);
    default: return hipErrorInvalidValue;
  }
}
