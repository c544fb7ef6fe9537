// Decode attention against a left-aligned KV cache ("Gemma 3 Attention
// Block", How it works: the step's K and V land in the cache at the query's
// position; the query then attends to cached positions s <= pos, and on local
// layers only to s > pos - W; softmax over those slots mixes V).
//
// HBM-bound split-KV evaluation of that softmax:
//  * The allowed slot range [lo, pos] of row b is cut into chunks of C slots.
//    One workgroup streams one (row, chunk, KV head): K and V rows of that
//    head, d_h contiguous elements per slot, 16-byte loads, each byte read once
//    for all the query heads of the GQA group, in double-buffered rounds (the
//    next round's loads are in flight while this one is computed).
//  * The workgroup forms its queries itself from the raw projections
//    (RMSNorm with (1 + gamma), RoPE, alpha: "QK-Norm", How it works) while
//    its first round of loads is in flight; the workgroup whose chunk ends at
//    the row's position also forms the step's own key and value, writes them to
//    that cache slot and uses them there.
//  * Inside a wave, d_h/16 lanes share one slot (16 channels each); per-slot
//    logits are a short DPP sum. Each slot group keeps an online softmax state
//    (m, l, acc) per query head; groups and waves are merged by log-sum-exp,
//    and the chunk's (acc, m, l) go to the workspace.
//  * A second kernel merges the chunks of each (row, head) the same way, one
//    channel per thread, and divides by the total weight. Logits are in log2
//    units (q pre-scaled by log2 e), so every exponential is an exp2.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace {

// threads of a partial workgroup: 4 waves, or 8 on sliding-window layers
// (bf16, at most two query heads per workgroup), whose few workgroups (one
// per (row, chunk, KV head group), about one per CU) then keep twice the
// loads in flight (the 12B-like local attention stage 38.3 -> 37.2 us; the
// many-workgroup global layer is slower so)
constexpr int kDecThreadsGlobal = 256, kDecThreadsLocal = 512;
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
// The workgroup forms its own queries from the raw projections (QK-norm,
// RoPE, alpha), and the workgroup whose chunk ends at the row's position also
// forms the step's own key and value, writes them to that cache slot (head
// group 0 only) and uses them for that slot. The first round of cache loads is
// issued before this set-up, so its latency hides the norm and RoPE work.
template <typename T, int D, int GQ, int kDecThreads>
__global__ void __launch_bounds__(kDecThreads)
decode_attn_partial(const float *__restrict__ qkv, const T *__restrict__ gamma_q,
                    const T *__restrict__ gamma_k, T *__restrict__ k_cache,
                    T *__restrict__ v_cache, const int32_t *__restrict__ pos,
                    float *__restrict__ part, DecodeArgs a, int n_hgrp) {
  constexpr int LPS = D / kChansPerLane;         // lanes per slot
  constexpr int kGroupsPerWave = kWave / LPS;
  constexpr int kWaves = kDecThreads / kWave;
  constexpr int NG = kGroupsPerWave * kWaves;
  constexpr int kHalf = D / 2;
  constexpr int kVec = GQ + 2;                   // query heads, the step's key, its value
  __shared__ float red[kWaves][GQ][D + 2];
  __shared__ float raw[kVec][D];                 // raw projections, then finished queries
  __shared__ float ssq[kVec];
  __shared__ float2 rot[kHalf];                  // (cos, sin) of each channel pair
  __shared__ __attribute__((aligned(16))) T kv_new[2][D];  // the step's key and value, as cached

  const int chunk = blockIdx.x, b = blockIdx.y;
  const int kh = blockIdx.z / n_hgrp, hgrp = blockIdx.z % n_hgrp;
  const int G = a.H / a.Hk;
  const int h0 = kh * G + hgrp * GQ;
  int lo, hi;
  row_range(pos, b, a.S, a.local, a.window, lo, hi);
  const int c_lo = lo + chunk * a.chunk;
  if (c_lo > hi) return;  // chunk past this row's range (uniform per block)
  const int c_hi = min(hi, c_lo + a.chunk - 1);
  const bool has_new = c_hi == hi;  // this chunk ends at the row's position

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sub = lane % LPS;             // which 16-channel slice
  const int grp = wave * kGroupsPerWave + lane / LPS;

  const size_t slot_stride = (size_t)a.Hk * D;
  const T *kb = k_cache + ((size_t)b * a.S) * slot_stride + (size_t)kh * D;
  const T *vb = v_cache + ((size_t)b * a.S) * slot_stride + (size_t)kh * D;

  // Rounds of kDecUnroll slots per slot group, double-buffered: the loads of
  // round r + 1 are in flight while round r is computed, so each wave keeps
  // streaming from HBM without a gap per round.
  struct Round {
    Slice<T> k[kDecUnroll], v[kDecUnroll];
    bool ok[kDecUnroll];
  };
  Round buf[2];
  constexpr int kStep = NG * kDecUnroll;  // slots of one round of the workgroup
  auto issue = [&](Round &r, int s_base) {
#pragma unroll
    for (int u = 0; u < kDecUnroll; ++u) {
      const int s = s_base + u * NG;
      r.ok[u] = s <= c_hi;
      if (r.ok[u]) {
        r.k[u].template load<LPS>(kb + (size_t)s * slot_stride, sub);
        r.v[u].template load<LPS>(vb + (size_t)s * slot_stride, sub);
      } else {
        r.k[u].zero();
        r.v[u].zero();
      }
    }
  };
  const int s_first = c_lo + grp;
  issue(buf[0], s_first);

  // ---- queries (and the step's key / value) from the raw projections
  // ("QK-Norm", How it works: RMSNorm with (1 + gamma) over d_h, then RoPE,
  // then alpha; V is not normalised)
  const int n_qkv = (a.H + 2 * a.Hk) * D;
  const float *row = qkv + (size_t)b * n_qkv;
  const int n_vec = GQ + (has_new ? 2 : 0);
  for (int e = tid; e < n_vec * D; e += kDecThreads) {
    const int v = e / D, c = e % D;
    const int col = v < GQ ? (h0 + v) * D : v == GQ ? (a.H + kh) * D : (a.H + a.Hk + kh) * D;
    raw[v][c] = row[col + c];
  }
  if (tid < kHalf) {
    // theta^(-2i/d_h) = 2^(-(2i/d_h) log2 theta), in fp64
    const double inv_freq = exp2(-2.0 * (double)tid / (double)D * log2((double)a.theta));
    float c, sn;
    rope_sincos(hi, 1.0 / (double)a.scale, inv_freq, c, sn);
    rot[tid] = make_float2(c, sn);
  }
  __syncthreads();
  for (int v = wave; v < n_vec - (has_new ? 1 : 0); v += kWaves) {  // sums of squares (not V)
    float sq = 0.f;
#pragma unroll
    for (int c = lane; c < D; c += kWave) sq = fmaf(raw[v][c], raw[v][c], sq);
    sq = wave_sum(sq);
    if (lane == 0) ssq[v] = sq;
  }
  __syncthreads();
  const float q_mul = a.alpha * kLog2e;  // logits in log2 units: every exponential is an exp2
  for (int e = tid; e < (GQ + (has_new ? 1 : 0)) * kHalf; e += kDecThreads) {
    const int v = e / kHalf, i = e % kHalf;
    const bool is_q = v < GQ;
    const T *gam = is_q ? gamma_q : gamma_k;
    const float r = rsqrtf(ssq[v] / (float)D + 1e-6f);
    const float y1 = raw[v][i] * r * (1.f + to_f32(gam[i]));
    const float y2 = raw[v][i + kHalf] * r * (1.f + to_f32(gam[i + kHalf]));
    const float2 cs = rot[i];
    const float o1 = y1 * cs.x - y2 * cs.y, o2 = y2 * cs.x + y1 * cs.y;
    if (is_q) {
      raw[v][i] = o1 * q_mul;
      raw[v][i + kHalf] = o2 * q_mul;
    } else {
      kv_new[0][i] = from_f32<T>(o1);
      kv_new[0][i + kHalf] = from_f32<T>(o2);
    }
  }
  if (has_new)
    for (int c = tid; c < D; c += kDecThreads) kv_new[1][c] = from_f32<T>(raw[GQ + 1][c]);
  __syncthreads();
  if (has_new && hgrp == 0) {  // the cache write ("Gemma 3 Attention Block", Cache)
    T *kd = k_cache + ((size_t)b * a.S + hi) * slot_stride + (size_t)kh * D;
    T *vd = v_cache + ((size_t)b * a.S + hi) * slot_stride + (size_t)kh * D;
    for (int c = tid; c < D; c += kDecThreads) {
      kd[c] = kv_new[0][c];
      vd[c] = kv_new[1][c];
    }
  }

  float qv[GQ][kChansPerLane];
#pragma unroll
  for (int g = 0; g < GQ; ++g)
#pragma unroll
    for (int i = 0; i < kChansPerLane; ++i)
      qv[g][i] = raw[g][Slice<T>::template chan<LPS>(sub, i)];
  float m[GQ], l[GQ], acc[GQ][kChansPerLane];
#pragma unroll
  for (int g = 0; g < GQ; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int i = 0; i < kChansPerLane; ++i) acc[g][i] = 0.f;
  }

  auto compute = [&](Round &r, int s_base) {
    if (has_new) {  // the step's own slot: its key and value as just formed
#pragma unroll
      for (int u = 0; u < kDecUnroll; ++u)
        if (r.ok[u] && s_base + u * NG == hi) {
          r.k[u].template load<LPS>(kv_new[0], sub);
          r.v[u].template load<LPS>(kv_new[1], sub);
        }
    }
    float x[kDecUnroll][GQ];
#pragma unroll
    for (int u = 0; u < kDecUnroll; ++u)
#pragma unroll
      for (int g = 0; g < GQ; ++g) {
        float d = 0.f;
#pragma unroll
        for (int i = 0; i < kChansPerLane; ++i) d = fmaf(qv[g][i], r.k[u].get(i), d);
        d = group_sum_dpp<LPS>(d);
        x[u][g] = r.ok[u] ? d : -INFINITY;
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
          acc[g][i] = fmaf(x[u][g], r.v[u].get(i), acc[g][i]);
  };
  // rounds alternate between the two buffers (compile-time indices)
  for (int s_base = s_first; s_base <= c_hi; s_base += 2 * kStep) {
    if (s_base + kStep <= c_hi) issue(buf[1], s_base + kStep);
    compute(buf[0], s_base);
    if (s_base + kStep > c_hi) break;
    if (s_base + 2 * kStep <= c_hi) issue(buf[0], s_base + 2 * kStep);
    compute(buf[1], s_base + kStep);
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

// grid: x = H, y = B; CG x D threads: channel c of chunk group cg (chunks
// j with j mod CG = cg). Every thread loads, for a batch of up to
// kCombineBatch of its chunks at once, each chunk's (m, l) (the same
// addresses across the group) and its own channel of each partial, then
// merges them by log-sum-exp with a running maximum: one round trip per batch.
// With CG > 1 the groups' (M, sum, l) meet in LDS and group 0 merges them
// the same way (long rows: 128 chunks take two round trips, not eight).
constexpr int kMaxChunks = 128;  // decode_chunk keeps every row at <= 128 chunks
constexpr int kCombineBatch = 16;

template <typename T, int D, int CG>
__global__ void __launch_bounds__(D * CG)
decode_attn_combine(const float *__restrict__ part, const int32_t *__restrict__ pos,
                    T *__restrict__ o, DecodeArgs a) {
  const int h = blockIdx.x, b = blockIdx.y, c = threadIdx.x % D, cg = threadIdx.x / D;
  int lo, hi;
  row_range(pos, b, a.S, a.local, a.window, lo, hi);
  const int n = hi >= lo ? div_up(hi - lo + 1, a.chunk) : 0;
  const float *pp = part + ((size_t)b * a.H + h) * a.n_chunks * (D + 2);
  float M = -INFINITY, sa = 0.f, sl = 0.f;
  for (int j = cg; j < n; j += CG * kCombineBatch) {
    float mv[kCombineBatch], lv[kCombineBatch], v[kCombineBatch];
#pragma unroll
    for (int u = 0; u < kCombineBatch; ++u) {
      const int jj = j + CG * u;
      const bool ok = jj < n;
      const float *pj = pp + (size_t)(ok ? jj : 0) * (D + 2);
      const float2 ml = *reinterpret_cast<const float2 *>(pj + D);
      mv[u] = ok ? ml.x : -INFINITY;
      lv[u] = ml.y;
      v[u] = pj[c];
    }
    float mb = M;
#pragma unroll
    for (int u = 0; u < kCombineBatch; ++u) mb = fmaxf(mb, mv[u]);
    // every chunk holds at least one allowed slot, so mb is finite
    const float corr = exp2f(M - mb);
    sa *= corr;
    sl *= corr;
#pragma unroll
    for (int u = 0; u < kCombineBatch; ++u) {
      const float wj = exp2f(mv[u] - mb);  // 0 for the unused tail of a batch
      sa = fmaf(wj, v[u], sa);
      sl = fmaf(wj, lv[u], sl);
    }
    M = mb;
  }
  if constexpr (CG > 1) {
    __shared__ float red[3][CG][D];
    red[0][cg][c] = M;
    red[1][cg][c] = sa;
    red[2][cg][c] = sl;
    __syncthreads();
    if (cg != 0) return;
    float mb = M;
#pragma unroll
    for (int g = 1; g < CG; ++g) mb = fmaxf(mb, red[0][g][c]);
    if (mb == -INFINITY) {  // a row without chunks (position outside the cache)
      sa = 0.f;
      sl = 0.f;
    } else {
      sa = 0.f;
      sl = 0.f;
#pragma unroll
      for (int g = 0; g < CG; ++g) {
        const float wg = exp2f(red[0][g][c] - mb);  // 0 for a group without chunks
        sa = fmaf(wg, red[1][g][c], sa);
        sl = fmaf(wg, red[2][g][c], sl);
      }
    }
  }
  o[((size_t)b * a.H + h) * D + c] = from_f32<T>(sl > 0.f ? sa / sl : 0.f);
}

template <typename T, int D, int GQ>
hipError_t launch_dec(const float *qkv, const T *gq, const T *gk, T *kc, T *vc,
                      const int32_t *pos, float *part, T *o, const DecodeArgs &a, hipStream_t s) {
  const int G = a.H / a.Hk;
  const int n_hgrp = G / GQ;
  dim3 grid(a.n_chunks, a.B, a.Hk * n_hgrp);
  // (8 waves only where a wave's registers fit two waves per SIMD: bf16 and
  // at most two query heads per workgroup)
  constexpr bool kWide = std::is_same<T, bf16>::value && GQ <= 2;
  bool launched = false;
  if constexpr (kWide) {
    if (a.local) {
      hipLaunchKernelGGL((decode_attn_partial<T, D, GQ, kDecThreadsLocal>), grid,
                         dim3(kDecThreadsLocal), 0, s, qkv, gq, gk, kc, vc, pos, part, a, n_hgrp);
      launched = true;
    }
  }
  if (!launched)
    hipLaunchKernelGGL((decode_attn_partial<T, D, GQ, kDecThreadsGlobal>), grid,
                       dim3(kDecThreadsGlobal), 0, s, qkv, gq, gk, kc, vc, pos, part, a, n_hgrp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // rows of many chunks: four chunk groups per (row, head)
  if (a.n_chunks > 2 * kCombineBatch && D * 4 <= 1024)
    hipLaunchKernelGGL((decode_attn_combine<T, D, 4>), dim3(a.H, a.B), dim3(D * 4), 0, s, part,
                       pos, o, a);
  else
    hipLaunchKernelGGL((decode_attn_combine<T, D, 1>), dim3(a.H, a.B), dim3(D), 0, s, part, pos,
                       o, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_dec_g(const float *qkv, const T *gq, const T *gk, T *kc, T *vc,
                        const int32_t *pos, float *part, T *o, const DecodeArgs &a,
                        hipStream_t s) {
  const int G = a.H / a.Hk;
  if (G % 4 == 0) return launch_dec<T, D, 4>(qkv, gq, gk, kc, vc, pos, part, o, a, s);
  if (G % 2 == 0) return launch_dec<T, D, 2>(qkv, gq, gk, kc, vc, pos, part, o, a, s);
  return launch_dec<T, D, 1>(qkv, gq, gk, kc, vc, pos, part, o, a, s);
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
  // a workgroup streams rounds of 16 slot groups x kDecUnroll slots; a
  // local row's window splits into two chunks (at least 256 slots), so the
  // W = 1024 window of a (row, KV head group) is 2 workgroups and the whole
  // step fits one wave of resident workgroups, each paying its query set-up
  // once (measured on the 12B-like local step: 71.4 us against 72.6 with
  // 4 chunks of 256 and 80.5 with one of 1024)
  int c = local && window < S ? max(256, div_up_h(window, 2 * 64) * 64) : 256;
  while (div_up_h(range, c) > kMaxChunks) c *= 2;
  return c;
}

template <typename T>
hipError_t launch_decode_attn(const float *qkv, const T *gamma_q, const T *gamma_k, T *k_cache,
                              T *v_cache, const int32_t *pos, float *part, T *o,
                              const DecodeArgs &a, hipStream_t s) {
  switch (a.d_h) {
    case 64: return launch_dec_g<T, 64>(qkv, gamma_q, gamma_k, k_cache, v_cache, pos, part, o, a, s);
    case 128:
      return launch_dec_g<T, 128>(qkv, gamma_q, gamma_k, k_cache, v_cache, pos, part, o, a, s);
    case 256:
      return launch_dec_g<T, 256>(qkv, gamma_q, gamma_k, k_cache, v_cache, pos, part, o, a, s);
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

template hipError_t launch_decode_attn<bf16>(const float *, const bf16 *, const bf16 *, bf16 *,
                                             bf16 *, const int32_t *, float *, bf16 *,
                                             const DecodeArgs &, hipStream_t);
template hipError_t launch_decode_attn<float>(const float *, const float *, const float *, float *,
                                              float *, const int32_t *, float *, float *,
                                              const DecodeArgs &, hipStream_t);
template hipError_t launch_splitk_reduce<bf16>(const float *, int, bf16 *, long, hipStream_t);
template hipError_t launch_splitk_reduce<float>(const float *, int, float *, long, hipStream_t);
