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
//  * Softmax reference max m is only raised when a logit exceeds it by more
//    than 8 (log2 units), so exp2 arguments stay <= 8 and the O/l rescale is
//    skipped for the whole wave on most tiles. The result is unchanged: l and
//    O share the same reference, which cancels in O / l.
//  * Tiles move global -> LDS with direct loads (global_load_lds, 16 bytes
//    per lane, no staging registers) into XOR-swizzled, unpadded layouts that
//    keep the fragment reads free of bank conflicts. K runs one tile ahead of
//    V: while the softmax of tile i runs on the vector ALUs, the S MFMAs of
//    tile i+1 are already queued, so the matrix pipe does not wait for it.
//    K and V^T are each double-buffered; one barrier per tile.
//  * Split-KV: when (rows x heads) give too few workgroups to fill the chip,
//    the key range of each query tile is cut into chunks handled by separate
//    workgroups; a query tile with several chunks writes normalised partial
//    outputs with their (m, l), merged by flash_combine.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace {

constexpr int kBN = 64;       // keys per tile
constexpr int kThreads = 256; // 4 waves
constexpr int kRowsPerWave = 32;
constexpr float kRescaleSlack = 8.f;  // log2 units

template <int D> struct AttnCfg {
  // S of tile i+1 is issued before the softmax of tile i (needs a second S
  // register set; at d_h = 256 that no longer fits beside O and Q).
  static constexpr bool kPipeS = D <= 128;
  static constexpr int kKRowBytes = 2 * D;            // one key row of K
  static constexpr int kKChunks = D / 8;              // 16-byte chunks per K row
  static constexpr int kKTileBytes = kBN * kKRowBytes;
  static constexpr int kVRowBytes = 2 * kBN;          // one channel row of V^T (128 B)
  static constexpr int kVTileBytes = D * kVRowBytes;
  static constexpr int kLdsBytes = 2 * kKTileBytes + 2 * kVTileBytes;
  static constexpr int kKLoads = kKTileBytes / 1024 / 4;  // 1 KB loads per wave per K tile
  static constexpr int kVLoads = kVTileBytes / 1024 / 4;
  static constexpr int kKS = D / 16;                      // k-steps of the QK^T contraction
  static constexpr int kDB = D / 32;                      // 32-row blocks of O^T
};

// XOR swizzles of the 16-byte chunk index inside a row. K fragment reads hit
// rows kappa(i) for 8 lanes at a time, i.e. rows {0,1,2,3,8,9,10,11} + const;
// V^T reads hit 8 consecutive rows. Both maps send those rows to 8 distinct
// chunk positions mod 8, so each 128-byte LDS access spans all banks.
DEVI int swz_k(int r) { return (r & 3) | ((r & 8) >> 1); }
DEVI int swz_v(int r) { return r & 7; }

// One direct global -> LDS load: each lane moves 16 bytes to lds + 16 * lane.
DEVI void load_lds16(const void *g, void *lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void *)lds_wave_base,
                                   16, 0, 0);
}

// Key permutation inside a 32-key block (see the header comment).
DEVI int kappa(int i) {
  const int g = i >> 3, h = (i >> 2) & 1, r = i & 3;
  return 16 * (g >> 1) + 8 * h + 4 * (g & 1) + r;
}

struct Geo {  // per-workgroup geometry, identical in the attention and combine kernels
  int b, kh, hgrp, qt, t_lo, t_hi, len, kv_begin, kv_end, tile_begin, n_active;
};

DEVI Geo geometry(const AttnArgs &a, const int32_t *kv_len, int base_id, int gp, int n_qtiles,
                  int n_hgrp, int chunk_keys) {
  Geo g;
  g.qt = n_qtiles - 1 - base_id % n_qtiles;  // longest (latest) query tile first
  int rest = base_id / n_qtiles;
  g.hgrp = rest % n_hgrp;
  rest /= n_hgrp;
  g.kh = rest % a.Hk;
  g.b = rest / a.Hk;
  const int TQ = kRowsPerWave * (4 / gp);
  g.t_lo = g.qt * TQ;
  g.t_hi = min(a.T, g.t_lo + TQ);
  g.len = kv_len ? kv_len[g.b] : a.T;
  g.kv_begin = a.local ? max(0, g.t_lo - a.window + 1) : 0;
  g.kv_end = min(g.t_hi, g.len);  // exclusive
  g.tile_begin = (g.kv_begin / kBN) * kBN;
  g.n_active = g.kv_end > g.kv_begin ? div_up(g.kv_end - g.tile_begin, chunk_keys) : 1;
  return g;
}

template <int D>
__global__ void __launch_bounds__(kThreads)
flash_attn_fwd_bf16(const bf16 *__restrict__ q, const bf16 *__restrict__ k,
                    const bf16 *__restrict__ vt, const int32_t *__restrict__ kv_len,
                    const bf16 *__restrict__ gamma_k, bf16 *__restrict__ o,
                    bf16 *__restrict__ part_o, float *__restrict__ part_ml, AttnArgs a, int gp,
                    int n_qtiles, int n_hgrp, int n_split, int chunk_keys) {
  using Cfg = AttnCfg<D>;
  extern __shared__ __attribute__((aligned(16))) bf16 lds[];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int G = a.H / a.Hk;
  // Logical order: (b, kh, head group) runs of query tiles (longest first),
  // the key chunks of one query tile adjacent; runs stay on one XCD.
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int split = bid % n_split;
  const Geo geo = geometry(a, kv_len, bid / n_split, gp, n_qtiles, n_hgrp, chunk_keys);
  if (split >= geo.n_active) return;  // uniform per block
  const int b = geo.b, kh = geo.kh;

  const int wpg = 4 / gp;  // waves per query head
  const int hg = w / wpg, tb = w % wpg;
  const int h = kh * G + geo.hgrp * gp + hg;
  const int wq0 = geo.t_lo + tb * kRowsPerWave;   // first query row of this wave
  const int wq_last = min(wq0 + kRowsPerWave, a.T) - 1;
  const int len = geo.len;
  const int t_lo = geo.t_lo, t_hi = geo.t_hi;

  const int my_begin = geo.tile_begin + split * chunk_keys;
  const int my_end = geo.kv_end > geo.kv_begin ? min(geo.kv_end, my_begin + chunk_keys) : my_begin;

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
  float m_ref = -INFINITY, l_run = 0.f;

  const char *kbase = (const char *)(k + ((size_t)b * a.Hk + kh) * a.T_pad * D);
  const char *vbase = (const char *)(vt + ((size_t)b * a.Hk + kh) * D * a.T_pad);
  auto kbuf = [&](int i) { return (char *)lds + i * Cfg::kKTileBytes; };
  auto vbuf = [&](int i) { return (char *)lds + 2 * Cfg::kKTileBytes + i * Cfg::kVTileBytes; };

  // Wave w fills 1 KB pieces w, w + 4, ... of a tile. Lane l of piece j writes
  // byte 16 l of it: K row r, chunk position p holds logical chunk p ^ swz_k(r).
  auto issue_k = [&](int s0, char *dst) {
#pragma unroll
    for (int i = 0; i < Cfg::kKLoads; ++i) {
      const int piece = w + 4 * i;
      const int byte = piece * 1024 + 16 * lane;
      const int r = byte / Cfg::kKRowBytes, pch = (byte % Cfg::kKRowBytes) / 16;
      const int cch = pch ^ swz_k(r);
      load_lds16(kbase + (size_t)(s0 + r) * Cfg::kKRowBytes + 16 * cch, dst + piece * 1024);
    }
  };
  auto issue_v = [&](int s0, char *dst) {
#pragma unroll
    for (int i = 0; i < Cfg::kVLoads; ++i) {
      const int piece = w + 4 * i;
      const int byte = piece * 1024 + 16 * lane;
      const int r = byte / Cfg::kVRowBytes, pch = (byte % Cfg::kVRowBytes) / 16;
      const int cch = pch ^ swz_v(r);
      load_lds16(vbase + (size_t)r * a.T_pad * 2 + (size_t)s0 * 2 + 16 * cch, dst + piece * 1024);
    }
  };

  const int n_tiles = my_end > my_begin ? div_up(my_end - my_begin, kBN) : 0;
  if (n_tiles > 0) {
    issue_k(my_begin, kbuf(0));
    issue_v(my_begin, vbuf(0));
    if (Cfg::kPipeS && n_tiles > 1) issue_k(my_begin + kBN, kbuf(1));
  }
  // The barrier waits for every outstanding load (Q fragments, first tiles),
  // so inside the loop only the newest prefetches are ever pending.
  __syncthreads();

  const int krow = kappa(col);  // permuted key row this lane feeds
  auto wave_live = [&](int s0) {  // does any row of this wave see a key of the tile?
    return s0 <= wq_last && !(a.local && s0 + kBN - 1 <= wq0 - a.window);
  };
  // S^T for the tile in kbuf: two 32-key blocks, reads batched ahead of MFMAs.
  auto qk = [&](const char *kb_lds, f32x16 (&acc_s)[2]) {
    constexpr int kBatch = Cfg::kKS < 8 ? Cfg::kKS : 8;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      acc_s[kb] = f32x16{};
      const int r = 32 * kb + krow;
      const char *rowp = kb_lds + r * Cfg::kKRowBytes;
      const int sw = swz_k(r);
#pragma unroll
      for (int k0 = 0; k0 < Cfg::kKS; k0 += kBatch) {
        bf16x8 kf[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j)
          kf[j] = *reinterpret_cast<const bf16x8 *>(rowp + 16 * ((2 * (k0 + j) + hh) ^ sw));
#pragma unroll
        for (int j = 0; j < kBatch; ++j)
          acc_s[kb] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[j], qf[k0 + j], acc_s[kb], 0, 0, 0);
      }
    }
  };

  // Fixed softmax reference. |logit| <= |q_t| |k_s| (Cauchy-Schwarz) and a
  // key after RMSNorm has |k| <= sqrt(d_h) max_c |1 + gamma_k[c]|, so
  // U_t = |q_t| sqrt(d_h) max|1 + gamma_k| bounds every logit of row t:
  // p = exp2((x - U_t) log2 e) <= 1 never overflows and the running max and
  // its rescale of O disappear. While 2 U_t log2 e <= 100 the row's largest p
  // is >= 2^-100, far from underflow; otherwise the workgroup takes the
  // running-max path below.
  __shared__ float red4[4];
  float gmax = 0.f;
  for (int c = tid; c < D; c += kThreads) gmax = fmaxf(gmax, fabsf(1.f + (float)gamma_k[c]));
  gmax = wave_max(gmax);
  if (lane == 0) red4[w] = gmax;
  __syncthreads();
  gmax = fmaxf(fmaxf(red4[0], red4[1]), fmaxf(red4[2], red4[3]));
  float qq = 0.f;
#pragma unroll
  for (int ks = 0; ks < Cfg::kKS; ++ks)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float v = (float)qf[ks][j];
      qq = fmaf(v, v, qq);
    }
  qq += __shfl_xor(qq, 32, kWave);
  // 1% margin covers the bf16 rounding of the stored keys
  const float m_fixed = sqrtf(qq) * sqrtf((float)D) * gmax * 1.01f * kLog2e;
  const bool fixed_ok = __syncthreads_and(2.f * m_fixed <= 100.f);

  auto run = [&](auto fixed_tag) {
    constexpr bool kFixed = decltype(fixed_tag)::value;
    f32x16 s_cur[2], s_next[2];
    if (Cfg::kPipeS && n_tiles > 0 && wave_live(my_begin)) qk(kbuf(0), s_cur);
    if (kFixed) m_ref = m_fixed;

    for (int it = 0; it < n_tiles; ++it) {
      const int s0 = my_begin + it * kBN;
      const int cur = it & 1, nxt = cur ^ 1;
      // prefetch. Pipelined: K of tile it+2 into the K buffer tile `it` used
      // (its S was formed last iteration); otherwise K of tile it+1. V of it+1.
      if (Cfg::kPipeS) {
        if (it + 2 < n_tiles) issue_k(s0 + 2 * kBN, kbuf(cur));
      } else if (it + 1 < n_tiles) {
        issue_k(s0 + kBN, kbuf(nxt));
      }
      if (it + 1 < n_tiles) issue_v(s0 + kBN, vbuf(nxt));
      // S of the next tile goes to the matrix pipe before this tile's softmax
      if (Cfg::kPipeS) {
        if (it + 1 < n_tiles && wave_live(s0 + kBN)) qk(kbuf(nxt), s_next);
      } else if (wave_live(s0)) {
        qk(kbuf(cur), s_cur);
      }

      if (wave_live(s0)) {
        // tile-uniform mask decision for the whole workgroup
        const bool full = (s0 + kBN - 1 <= t_lo) && (s0 + kBN - 1 < len) &&
                          (!a.local || s0 >= t_hi - a.window);
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            float x = s_cur[kb][e];
            if (!full) {
              const int g = e >> 2, r = e & 3;
              const int s = s0 + 32 * kb + 16 * (g >> 1) + 8 * hh + 4 * (g & 1) + r;
              const bool ok = s <= my_t && s < len && (!a.local || s > my_t - a.window);
              x = ok ? x : -INFINITY;
            }
            s_cur[kb][e] = x;
            if (!kFixed) mx = fmaxf(mx, x);
          }
        if (!kFixed) {
          mx = fmaxf(mx, __shfl_xor(mx, 32, kWave)) * kLog2e;
          const bool need = mx > m_ref + kRescaleSlack;
          if (__ballot(need)) {  // raise the reference (rare after the first tiles)
            const float m_new = need ? mx : m_ref;
            const float corr =
                m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_ref - m_new);
            m_ref = m_new;
            l_run *= corr;
#pragma unroll
            for (int db = 0; db < Cfg::kDB; ++db) acc_o[db] *= corr;
          }
        }
        const float neg_m = m_ref == -INFINITY ? 0.f : -m_ref;
        bf16x8 pf[4];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            pf[2 * kb + (e >> 3)][e & 7] =
                (bf16)__builtin_amdgcn_exp2f(fmaf(s_cur[kb][e], kLog2e, neg_m));
        // l sums the bf16-rounded weights the PV MFMAs use, so numerator and
        // denominator of O / l carry the same rounding
        float psum = 0.f;
        const bf16x2 ones = {(bf16)1.f, (bf16)1.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const u32x4 wv = __builtin_bit_cast(u32x4, pf[kk]);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t pair = wv[j];
            psum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair), ones, psum,
                                                   false);
          }
        }
        l_run += psum;

        const char *vb_lds = vbuf(cur);
#pragma unroll
        for (int db0 = 0; db0 < Cfg::kDB; db0 += 2) {
          bf16x8 vf[2][4];
#pragma unroll
          for (int d2 = 0; d2 < 2; ++d2) {
            const int r = 32 * (db0 + d2) + col;
            const char *rowp = vb_lds + r * Cfg::kVRowBytes;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
              vf[d2][kk] =
                  *reinterpret_cast<const bf16x8 *>(rowp + 16 * ((2 * kk + hh) ^ swz_v(r)));
          }
#pragma unroll
          for (int d2 = 0; d2 < 2; ++d2)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
              acc_o[db0 + d2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  vf[d2][kk], pf[kk], acc_o[db0 + d2], 0, 0, 0);
        }
      }
      // the barrier also waits for this iteration's prefetches to land
      __syncthreads();
      if (Cfg::kPipeS) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) s_cur[kb] = s_next[kb];
      }
    }
  };
  if (fixed_ok)
    run(std::integral_constant<bool, true>{});
  else
    run(std::integral_constant<bool, false>{});

  // Normalise; write the output row (single chunk) or a partial (several chunks).
  const float l_tot = l_run + __shfl_xor(l_run, 32, kWave);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (my_t >= a.T) return;
  bf16 *op;
  if (geo.n_active == 1) {
    op = o + ((size_t)b * a.T + my_t) * ((size_t)a.H * D) + (size_t)h * D;
  } else {
    const size_t row = (((size_t)split * a.B + b) * a.H + h) * a.T + my_t;
    op = part_o + row * D;
    if (hh == 0) {
      part_ml[2 * row] = m_ref;
      part_ml[2 * row + 1] = l_tot;
    }
  }
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

// Merge the key chunks of query tiles that had more than one:
// o = sum_j 2^(m_j - M) l_j o_j / sum_j 2^(m_j - M) l_j. One wave per output
// row (b, h, t); rows whose query tile had a single chunk were written by the
// attention kernel and are skipped.
template <int D>
__global__ void __launch_bounds__(256)
flash_combine(const int32_t *__restrict__ kv_len, bf16 *__restrict__ o,
              const bf16 *__restrict__ part_o, const float *__restrict__ part_ml, AttnArgs a,
              int gp, int n_qtiles, int n_hgrp, int n_split, int chunk_keys) {
  constexpr int kPer = D / 64;  // channels per lane
  const int lane = threadIdx.x & 63;
  const long row_id = (long)blockIdx.x * 4 + (threadIdx.x >> 6);  // over B*H*T
  if (row_id >= (long)a.B * a.H * a.T) return;
  const int t = (int)(row_id % a.T);
  const int h = (int)((row_id / a.T) % a.H);
  const int b = (int)(row_id / ((long)a.T * a.H));
  const int G = a.H / a.Hk;
  const int kh = h / G, hgrp = (h % G) / gp;
  const int qt = t / (kRowsPerWave * (4 / gp));
  const int base_id = ((b * a.Hk + kh) * n_hgrp + hgrp) * n_qtiles + (n_qtiles - 1 - qt);
  const Geo geo = geometry(a, kv_len, base_id, gp, n_qtiles, n_hgrp, chunk_keys);
  if (geo.n_active <= 1) return;

  // every load of the row is issued before any arithmetic (n_active <= 8)
  float mj[8], lj[8], oj[8][kPer];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    mj[j] = -INFINITY;
    lj[j] = 0.f;
#pragma unroll
    for (int i = 0; i < kPer; ++i) oj[j][i] = 0.f;
    if (j < geo.n_active) {
      const size_t row = (((size_t)j * a.B + b) * a.H + h) * a.T + t;
      mj[j] = part_ml[2 * row];
      lj[j] = part_ml[2 * row + 1];
#pragma unroll
      for (int i = 0; i < kPer; ++i) oj[j][i] = (float)part_o[row * D + lane * kPer + i];
    }
  }
  float M = -INFINITY;
#pragma unroll
  for (int j = 0; j < 8; ++j) M = fmaxf(M, mj[j]);
  const float mu = M == -INFINITY ? 0.f : M;
  float num[kPer] = {}, den = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float wl = j < geo.n_active ? exp2f(mj[j] - mu) * lj[j] : 0.f;
    den += wl;
#pragma unroll
    for (int i = 0; i < kPer; ++i) num[i] = fmaf(wl, oj[j][i], num[i]);
  }
  bf16 *op = o + ((size_t)b * a.T + t) * ((size_t)a.H * D) + (size_t)h * D + lane * kPer;
#pragma unroll
  for (int i = 0; i < kPer; ++i) op[i] = (bf16)(den > 0.f ? num[i] / den : 0.f);
}

struct Plan {
  int gp, n_qtiles, n_hgrp, n_split, chunk_keys;
  long n_base;
};

Plan plan(const AttnArgs &a) {
  Plan p;
  const int G = a.H / a.Hk;
  p.gp = (G % 4 == 0) ? 4 : (G % 2 == 0) ? 2 : 1;
  const int TQ = kRowsPerWave * (4 / p.gp);
  p.n_qtiles = div_up_h(a.T, TQ);
  p.n_hgrp = G / p.gp;
  p.n_base = (long)a.B * a.Hk * p.n_hgrp * p.n_qtiles;
  // Split only when one query tile's key range is much longer than the
  // average per-CU load (one 131 KB-LDS workgroup per CU): the critical path
  // then sits in a few long workgroups. Chunks cost a per-workgroup prologue
  // and a merge, so aim at about twice the average load per chunk
  // (measured on the 1B shape: local layer best unsplit, global best 2-way).
  const int TQ2 = kRowsPerWave * (4 / p.gp);
  const int max_keys = a.local ? min(a.T, TQ2 + a.window - 1) : a.T;
  const int max_tiles = div_up_h(max_keys, kBN) + 1;
  // key tiles over all query tiles of one (b, kh, head group), closed form
  const double total_tiles =
      a.local ? p.n_qtiles * (max_keys / (double)kBN + 1.0)
              : p.n_qtiles * ((a.T + TQ2) / 2.0 / kBN + 1.0);
  const double avg = total_tiles * (double)(p.n_base / p.n_qtiles) / 256.0;
  p.n_split = 1;
  if (max_tiles > 3.0 * avg && avg > 0) {
    p.n_split = (int)((max_tiles + 2 * avg - 1) / (2 * avg));
    if (p.n_split > 8) p.n_split = 8;  // flash_combine merges at most 8 chunks
    if (p.n_split < 1) p.n_split = 1;
  }
  // one chunk covers every key range when there is no split
  p.chunk_keys = p.n_split == 1 ? a.T + kBN : div_up_h(max_tiles, p.n_split) * kBN;
  return p;
}

template <int D>
hipError_t launch_d(const bf16 *q, const bf16 *k, const bf16 *vt, const int32_t *kv_len,
                    const bf16 *gamma_k, bf16 *o, bf16 *part_o, float *part_ml, const AttnArgs &a,
                    hipStream_t s) {
  using Cfg = AttnCfg<D>;
  const Plan p = plan(a);
  hipError_t e = hipFuncSetAttribute((const void *)flash_attn_fwd_bf16<D>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     Cfg::kLdsBytes);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(flash_attn_fwd_bf16<D>, dim3((unsigned)(p.n_base * p.n_split)),
                     dim3(kThreads), Cfg::kLdsBytes, s, q, k, vt, kv_len, gamma_k, o, part_o,
                     part_ml, a,
                     p.gp, p.n_qtiles, p.n_hgrp, p.n_split, p.chunk_keys);
  e = hipGetLastError();
  if (e != hipSuccess || p.n_split == 1) return e;
  const long rows = (long)a.B * a.H * a.T;
  hipLaunchKernelGGL(flash_combine<D>, dim3((unsigned)div_up_h(rows, 4)), dim3(256), 0, s, kv_len,
                     o, part_o, part_ml, a, p.gp, p.n_qtiles, p.n_hgrp, p.n_split, p.chunk_keys);
  return hipGetLastError();
}

}  // namespace

size_t flash_attn_partial_bytes(const AttnArgs &a) {
  const Plan p = plan(a);
  if (p.n_split == 1) return 0;
  return (size_t)p.n_split * a.B * a.H * a.T * ((size_t)a.d_h * 2 + 8);
}

hipError_t launch_flash_attn_bf16(const bf16 *q, const bf16 *k, const bf16 *vt,
                                  const int32_t *kv_len, const bf16 *gamma_k, bf16 *o,
                                  void *partial, const AttnArgs &a, hipStream_t s) {
  const size_t rows = (size_t)plan(a).n_split * a.B * a.H * a.T;
  bf16 *part_o = (bf16 *)partial;
  float *part_ml = partial ? (float *)((char *)partial + rows * a.d_h * 2) : nullptr;
  switch (a.d_h) {
    case 64: return launch_d<64>(q, k, vt, kv_len, gamma_k, o, part_o, part_ml, a, s);
    case 128: return launch_d<128>(q, k, vt, kv_len, gamma_k, o, part_o, part_ml, a, s);
    case 256: return launch_d<256>(q, k, vt, kv_len, gamma_k, o, part_o, part_ml, a, s);
    default: return hipErrorInvalidValue;
  }
}
