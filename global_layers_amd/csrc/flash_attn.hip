// Prefill attention core on gfx950 MFMA ("Gemma 3 Attention Block", How it
// works: logits = sum_c Q[t,h,c] K[s,h/G,c] with the GQA reshape; causal and
// padding mask, times the sliding mask 1[s > t-W] 1[s < t+W] on local layers;
// blocked logits take the K_MASK fill; softmax over s; weights mix V).
//
// Exact tiled evaluation of that definition:
//  * Blocked logits get exactly zero weight, as K_MASK does in fp32 whenever a
//    row has an allowed key; the fill value itself is never formed. Tiles that
//    no row of the workgroup may see are never visited.
//  * One workgroup = 4 waves = 128 query rows of one KV head (64 with one
//    row block per wave): the query heads of a GQA group (up to 4) are packed
//    into the workgroup, so each K/V tile staged in LDS feeds every query
//    head that reads it. At d_h <= 128 two workgroups share each CU
//    (registers capped at 256 per lane).
//  * A wave owns 32 query rows as two blocks of 16 (one block where two
//    would leave half the chip idle) and computes S^T = K Q^T with 16x16x32
//    bf16 MFMAs (gfx950 sustains a higher shader clock on them than on
//    32x32x16 ones: 2.2-2.3 against 1.75-1.95 GHz measured under a dense
//    load). Each K fragment (16 keys x 32 channels) feeds every row block. Lane l owns query l % 16 of each block and, of every 32-key
//    half, the 8 keys 8 (l / 16) .. + 7: the K rows of a half are fed as two
//    16-key sub-tiles in the order pi(j, i) (sub-tile j, MFMA row i), so that
//    a lane's S^T accumulators of the two sub-tiles are, in register order,
//    the 16-byte B operand of the PV MFMA (O^T += V^T P^T over the 32 keys)
//    without moving data.
//  * V arrives transposed ([d_h][T]) so the PV A operand is a contiguous
//    16-byte LDS read.
//  * Softmax reference: a per-row upper bound of the logits from the query
//    and key norms, fixed for the whole row, so there is no running maximum
//    and no rescale of O (rows where that bound is too loose take the exact
//    row maxima from a first pass over their keys; at d_h <= 128 a wave
//    whose bounds are all small takes the reference 0, which lets its S
//    accumulators start from the MFMA's inline zero). l and O share the
//    reference, which cancels in O / l.
//  * Tiles move global -> LDS with direct loads (16 bytes per lane, no
//    staging registers) into XOR-swizzled, unpadded layouts that keep the
//    fragment reads free of bank conflicts. Each 64-key tile runs as two
//    32-key halves in one fixed sequence of groups of 4 fragments; the S
//    MFMAs of the next half overlap the softmax and PV of this one. K sits in
//    four 32-key slots and V^T in two tile buffers; one barrier per tile.
//  * Split-KV: when (rows x heads) give too few workgroups to fill the chip,
//    the key range of each query tile is cut into chunks handled by separate
//    workgroups; a query tile with several chunks writes normalised fp32
//    partial outputs with their (m, l), merged by flash_combine.
#include <climits>
#include <type_traits>
#include <utility>

#include "common.h"
#include "kernels.h"

namespace {

constexpr int kBN = 64;       // keys per tile
constexpr int kThreads = 256; // 4 waves

template <int D> struct AttnCfg {
  static constexpr int kKRowBytes = 2 * D;            // one key row of K
  static constexpr int kKHalfBytes = 32 * kKRowBytes; // 32 keys of K (one key block)
  static constexpr int kVRowBytes = 2 * kBN;          // one channel row of V^T (128 B)
  static constexpr int kVTileBytes = D * kVRowBytes;
  // four K half-tile slots and two V^T tiles
  static constexpr int kLdsBytes = 4 * kKHalfBytes + 2 * kVTileBytes;
  static constexpr int kKHalfLoads = kKHalfBytes / 1024 / 4;  // 1 KB loads per wave per K half
  static constexpr int kVLoads = kVTileBytes / 1024 / 4;      // per V tile
  static constexpr int kKS = D / 32;                          // 32-channel k-steps of QK^T
  static constexpr int kCB = D / 16;                          // 16-channel blocks of O^T
};

// K row of a 32-key half fed as MFMA row i (0..15) of sub-tile j (0, 1):
// lane l's accumulator rows 4 (l / 16) + r of sub-tile j are then keys
// 8 (l / 16) + 4 j + r of the half.
DEVI int pi_row(int j, int i) { return 8 * (i >> 2) + 4 * j + (i & 3); }

// XOR swizzles of the 16-byte chunk index inside a row. The LDS serves a
// 16-byte-per-lane read 16 lanes (256 bytes, all 64 banks) per cycle, so the
// 16 rows that lanes 16j .. 16j+15 read must land on 16 distinct 16-byte bank
// positions. K fragment reads of lanes 0-15 hit rows pi_row(j, 0..15), i.e.
// rows {0-3, 8-11, 16-19, 24-27} (+4 for j = 1); V^T reads hit 16
// consecutive rows.
//  * K rows of >= 256 bytes (d_h >= 128): position = chunk mod 16; XOR with
//    bits 0, 1, 3, 4 of r, which differ across such a row set;
//  * 128-byte rows (V^T, K at d_h = 64): position = 8 (r & 1) + chunk mod 8;
//    K: XOR with bits 1, 3, 4 of r; V^T: with (r >> 1) & 7.
template <int D> DEVI int swz_k(int r) {
  return D >= 128 ? ((r & 3) | ((r >> 1) & 12)) : (((r >> 1) & 1) | ((r >> 2) & 6));
}
DEVI int swz_v(int r) { return (r >> 1) & 7; }
// Key-major V tiles (cache mode): a transposing read touches, per 32 lanes,
// 8 key rows (8 (l / 16) + 0..3, + 4 for the second read) x 32 bytes. The
// 32-byte unit index within the row is XORed with a function of the key that
// differs across those 8 rows (d_h >= 128: rows of 256 B and more start in
// the same bank, 8 units per 256 B; d_h = 64: 128-byte rows, odd rows in the
// other half, 4 units per row). As a 16-byte chunk XOR: twice that.
template <int D> DEVI int swz_vc_unit(int r) {
  return D >= 128 ? ((r & 3) | ((r >> 1) & 4)) : (((r >> 1) & 1) | ((r >> 2) & 2));
}
template <int D> DEVI int swz_vc(int r) { return 2 * swz_vc_unit<D>(r); }

// s_waitcnt immediate (gfx9 encoding): vmcnt(0) and lgkmcnt(0), expcnt free.
constexpr int kWaitVmLgkm0 = 0x7 << 4;

// All of this wave's tile loads have landed; then every wave's have.
DEVI void publish_tiles() {
  __builtin_amdgcn_s_waitcnt(kWaitVmLgkm0);
  __syncthreads();
}

// f(integral_constant<int, 0>) ... f(integral_constant<int, N - 1>), so the body
// can use its index in constant expressions.
template <typename F, int... I>
DEVI void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F> DEVI void static_for(F &&f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Group schedule of one 64-key tile (see the tile step in the attention
// kernel): for each 32-key half, kNG groups of 4 K fragments (8 S MFMAs) then
// kPG groups of 4 V^T fragments (8 PV MFMAs).
template <int D, int kQB> struct TileSched {
  using Cfg = AttnCfg<D>;
  static constexpr int kNQ = 2 * kQB;            // weight quads of a half
  static constexpr int kG = 4;                   // fragments per group
  static constexpr int kNG = 2 * Cfg::kKS / kG;  // S groups per half
  static constexpr int kPG = Cfg::kCB / kG;      // PV groups per half
  static constexpr int kNGT = kNG + kPG;         // groups per half
  static constexpr int kPieces = 2 * Cfg::kKHalfLoads + Cfg::kVLoads;  // prefetch loads per tile
  static constexpr int kPPG = (kPieces + kNGT - 1) / kNGT;             // of them per first-half group
  // The 8 kQB weights of a lane's half (kNQ quads of 4: quad 2 b + j holds
  // row block b, sub-tile j) pass three stages: exp2, packing to bf16 (the PV
  // B operand of row block b), and the row sum of the packed values (l sums
  // the bf16-rounded weights the PV MFMAs use, so numerator and denominator
  // of O / l carry the same rounding). Exps of quad q and their packing sit
  // in S group q kNG / kNQ (every PV group takes all row blocks' operands, so
  // all packing precedes the first PV group; packing right after the exps
  // keeps the exponentials' registers short-lived), its sum one group later.
  static constexpr int e_grp(int qd) { return qd * kNG / kNQ; }
  static constexpr int c_grp(int qd) { return e_grp(qd); }
  static constexpr int d_grp(int qd) { return c_grp(qd) + 1 < kNGT ? c_grp(qd) + 1 : kNGT - 1; }
};

struct Geo {  // per-workgroup geometry, identical in the attention and combine kernels
  int b, kh, hgrp, qt, t_lo, t_hi, len, kv_begin, kv_end, tile_begin, n_active;
};

DEVI Geo geometry(const AttnArgs &a, const int32_t *kv_len, int base_id, int gp, int n_qtiles,
                  int n_hgrp, int chunk_keys, int rows_per_wave) {
  Geo g;
  g.qt = n_qtiles - 1 - base_id % n_qtiles;  // longest (latest) query tile first
  int rest = base_id / n_qtiles;
  g.hgrp = rest % n_hgrp;
  rest /= n_hgrp;
  g.kh = rest % a.Hk;
  g.b = rest / a.Hk;
  const int TQ = rows_per_wave * (4 / gp);
  g.t_lo = g.qt * TQ;  // query rows (absolute index: q0 + row)
  g.t_hi = min(a.T, g.t_lo + TQ);
  g.len = a.q0 + (kv_len ? kv_len[g.b] : a.T);  // keys below it are valid
  g.kv_begin = a.local ? max(0, a.q0 + g.t_lo - a.window + 1) : 0;
  g.kv_end = min(a.q0 + g.t_hi, g.len);  // exclusive
  g.tile_begin = (g.kv_begin / kBN) * kBN;
  g.n_active = g.kv_end > g.kv_begin ? div_up(g.kv_end - g.tile_begin, chunk_keys) : 1;
  return g;
}

// At d_h <= 128 the kernel is built for two waves per SIMD (256 registers per
// lane), so two workgroups share a CU and each one's barriers and
// post-barrier fragment waits fall while the other computes. At d_h = 256
// one wave per SIMD (O alone takes 128 registers).
// kCache: keys and values come straight from the caches ([B, S_cache, H_kv,
// d_h] each, V key-major, as a chunk of a longer prefill finds them). K rows
// land in LDS as in the workspace layout; a V tile lands key-major and the
// PV operand (8 consecutive keys of one channel per lane) is read with the
// transposing LDS read of gfx950 (two 4-key halves). Rows at or past the
// valid length are loaded as copies of the last valid row, so whatever the
// slots beyond it hold (NaN included) never reaches the arithmetic.
// kQB: 16-row query blocks per wave (two, or one for grids too small to fill
// the chip with two).
template <int D, bool kCache, int kQB>
__global__ void __launch_bounds__(kThreads, D <= 128 ? 2 : 1)
flash_attn_fwd_bf16(const bf16 *__restrict__ q, const bf16 *__restrict__ k,
                    const bf16 *__restrict__ vt, const int32_t *__restrict__ kv_len,
                    const bf16 *__restrict__ gamma_k, bf16 *__restrict__ o,
                    float *__restrict__ part_o, float *__restrict__ part_ml, AttnArgs a, int gp,
                    int n_qtiles, int n_hgrp, int n_split, int chunk_keys, int remap,
                    int ref_flags) {
  using Cfg = AttnCfg<D>;
  extern __shared__ __attribute__((aligned(16))) char lds[];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int G = a.H / a.Hk;
  // Logical order: (b, kh, head group) runs of query tiles (longest first),
  // the key chunks of one query tile adjacent; with `remap`, runs stay on one
  // XCD.
  const int bid = remap ? xcd_remap(blockIdx.x, gridDim.x) : (int)blockIdx.x;
  const int split = bid % n_split;
  constexpr int kRPW = 16 * kQB;  // query rows per wave
  const Geo geo = geometry(a, kv_len, bid / n_split, gp, n_qtiles, n_hgrp, chunk_keys, kRPW);
  if (split >= geo.n_active) return;  // uniform per block
  const int b = geo.b, kh = geo.kh;

  const int wpg = 4 / gp;  // waves per query head
  const int hg = w / wpg, tb = w % wpg;
  const int h = kh * G + geo.hgrp * gp + hg;
  const int wq0 = geo.t_lo + tb * kRPW;   // first query row of this wave
  const int len = geo.len;
  const int t_lo = geo.t_lo, t_hi = geo.t_hi;

  const int my_begin = geo.tile_begin + split * chunk_keys;
  const int my_end = geo.kv_end > geo.kv_begin ? min(geo.kv_end, my_begin + chunk_keys) : my_begin;

  const int qc = lane & 15, q4 = lane >> 4;  // query within a row block; key octet of a half
  int my_t[kQB];  // this lane's query row in each row block
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) my_t[qb] = wq0 + 16 * qb + qc;

  f32x4 acc_o[kQB][Cfg::kCB];
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
    for (int i = 0; i < Cfg::kCB; ++i) acc_o[qb][i] = f32x4{};
  float l_run[kQB];
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) l_run[qb] = 0.f;

  const char *kbase = kCache ? (const char *)(k + ((size_t)b * a.S_cache * a.Hk + kh) * D)
                             : (const char *)(k + ((size_t)b * a.Hk + kh) * a.T_pad * D);
  const char *vbase = kCache ? (const char *)(vt + ((size_t)b * a.S_cache * a.Hk + kh) * D)
                             : (const char *)(vt + ((size_t)b * a.Hk + kh) * D * a.T_pad);
  const uint32_t cache_pitch = (uint32_t)a.Hk * D * 2;  // bytes between cache slots

  const int n_tiles = my_end > my_begin ? div_up(my_end - my_begin, kBN) : 0;
  // Loads past the last tile are clamped to it: such a load only rewrites a
  // buffer that no later step reads.
  auto tile_s0 = [&](int t) { return my_begin + min(t, n_tiles - 1) * kBN; };
  // Wave w fills 1 KB pieces w, w + 4, ... of a buffer; lane l of piece j
  // writes byte 16 l of it. K half h (tile h / 2, key block h % 2) sits in
  // slot h % 4; its row r, chunk position p holds logical chunk p ^ swz_k(r).
  // Global addresses split into a wave-uniform base and a per-lane 32-bit
  // offset: one lane offset per K piece of a half (the K swizzle depends on
  // row bits 0-4, which differ between them), one for every V^T piece (pieces
  // 32 rows apart, which swz_v ignores).
  // With kCache a lane keeps its row within the piece and its chunk offset
  // instead; each load clamps the row to the last valid key and addresses it
  // from the tile's first row (wave-uniform base, 32-bit lane offset). A V
  // tile is then key-major: piece i holds keys 4 i (1024 / (2 d_h)) + ..., row
  // r with chunk position p holding logical chunk p ^ swz_vc(r); swz_vc
  // depends on row bits 0, 1 and 3, so pieces an odd multiple of 8 rows apart
  // (d_h = 256) take a second lane offset.
  const int wu = __builtin_amdgcn_readfirstlane(w);
  uint32_t k_lane[Cfg::kKHalfLoads];
  int k_row[Cfg::kKHalfLoads];
#pragma unroll
  for (int i = 0; i < Cfg::kKHalfLoads; ++i) {
    const int byte = (w + 4 * i) * 1024 + 16 * lane;
    const int r = byte / Cfg::kKRowBytes, pch = (byte % Cfg::kKRowBytes) / 16;
    k_lane[i] = (uint32_t)((kCache ? 0 : r * Cfg::kKRowBytes) + 16 * (pch ^ swz_k<D>(r)));
    k_row[i] = r;
  }
  constexpr int kVRowStep = 4096 / (2 * D);  // cache mode: key rows between a wave's V pieces
  uint32_t v_lane[2];
  int v_row;
  {
    const int byte = w * 1024 + 16 * lane;
    if constexpr (kCache) {
      const int r = byte / (2 * D), pch = (byte % (2 * D)) / 16;
#pragma unroll
      for (int p = 0; p < 2; ++p) v_lane[p] = (uint32_t)(16 * (pch ^ swz_vc<D>(r + p * kVRowStep)));
      v_row = r;
    } else {
      const int r = byte / Cfg::kVRowBytes, pch = (byte % Cfg::kVRowBytes) / 16;
      v_lane[0] = v_lane[1] = (uint32_t)(r * a.T_pad * 2 + 16 * (pch ^ swz_v(r)));
      v_row = 0;
    }
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)lds;
  // cache slot of key row s0 + r, clamped to the last valid key, as an offset from row s0
  auto clamped = [&](int s0, int r) { return (uint32_t)(min(s0 + r, len - 1) - s0) * cache_pitch; };
  // K rows 32 kbh .. 32 kbh + 31 of tile t into half slot `slot`
  auto issue_k_piece = [&](int t, int kbh, int slot, int i) {
    const uint32_t dst = lds0 + slot * Cfg::kKHalfBytes + (wu + 4 * i) * 1024;
    if constexpr (kCache) {
      const int s0 = tile_s0(t);
      load_lds16(kbase + (size_t)s0 * cache_pitch, clamped(s0, 32 * kbh + k_row[i]) + k_lane[i],
                 dst);
    } else {
      const char *src = kbase + (size_t)(tile_s0(t) + 32 * kbh) * Cfg::kKRowBytes;
      load_lds16(src, k_lane[i], dst);
    }
  };
  // V^T columns of tile t into V buffer `buf` (piece i: channel rows 32 i + ...),
  // or with kCache its key rows (piece i: rows 4 i (1024 / (2 d_h)) + ...)
  auto issue_v_piece = [&](int t, int buf, int i) {
    const uint32_t dst = lds0 + 4 * Cfg::kKHalfBytes + buf * Cfg::kVTileBytes + (wu + 4 * i) * 1024;
    if constexpr (kCache) {
      const int s0 = tile_s0(t);
      load_lds16(vbase + (size_t)s0 * cache_pitch,
                 clamped(s0, v_row + i * kVRowStep) + v_lane[i & 1], dst);
    } else {
      const char *src = vbase + (size_t)tile_s0(t) * 2 + (size_t)i * 32 * a.T_pad * 2;
      load_lds16(src, v_lane[0], dst);
    }
  };

  auto issue_prologue = [&]() {  // K halves 0, 1, 2 (slots 0-2) and V tile 0
    if (n_tiles <= 0) return;
#pragma unroll
    for (int h = 0; h < 3; ++h)
#pragma unroll
      for (int i = 0; i < Cfg::kKHalfLoads; ++i) issue_k_piece(h >> 1, h & 1, h, i);
#pragma unroll
    for (int i = 0; i < Cfg::kVLoads; ++i) issue_v_piece(0, 0, i);
  };
  // The first tiles go out before the Q fragments: the fragment selects below
  // wait for the Q data, and the tiles' loads then already overlap them.
  issue_prologue();
  // Q^T fragments (B operand): query my_t, channels 32 ks + 8 q4 + [0, 8).
  bf16x8 qf[kQB][Cfg::kKS];
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    const bool ok = my_t[qb] < a.T;
    const bf16 *qp = q + (((size_t)b * a.H + h) * a.T + (ok ? my_t[qb] : 0)) * D + 8 * q4;
#pragma unroll
    for (int ks = 0; ks < Cfg::kKS; ++ks)
      qf[qb][ks] = ok ? *reinterpret_cast<const bf16x8 *>(qp + 32 * ks) : bf16x8{};
  }

  // max_c |1 + gamma_k[c]| (bounds the key norms, below), every wave over all
  // d_h channels (no workgroup barrier for it); its loads, the Q fragments
  // and the first tiles are in flight together
  float gmax = 0.f;
#pragma unroll
  for (int c = lane; c < D; c += kWave) gmax = fmaxf(gmax, fabsf(1.f + (float)gamma_k[c]));
  // Every outstanding load (Q fragments, first tiles) lands before the loop,
  // so inside it only the newest prefetches are ever pending.
  publish_tiles();

  // Per-lane LDS byte offsets of the MFMA fragments. K: lane feeds row
  // pi_row(j, qc) of a 32-key half and reads logical chunk 4 ks + q4; the
  // swizzle flips chunk bits 0-3 (0-2 at d_h = 64), so one base per
  // (sub-tile, ks mod 4) and compile-time immediates cover every k-step. V^T:
  // row 16 cb + qc, chunk 4 kb + q4 (kb: the half); one base per half, cb in
  // the immediate.
  constexpr int kKSB = Cfg::kKS < 4 ? Cfg::kKS : 4;
  int koff[2][kKSB];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int krow = pi_row(j, qc), ksw = swz_k<D>(krow);
#pragma unroll
    for (int s = 0; s < kKSB; ++s) koff[j][s] = krow * Cfg::kKRowBytes + 16 * ((4 * s + q4) ^ ksw);
  }
  int voff[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
    voff[kb] = 4 * Cfg::kKHalfBytes + qc * Cfg::kVRowBytes + 16 * ((4 * kb + q4) ^ swz_v(qc));
  auto kfrag = [&](int slot, int j, int ks) {
    return *reinterpret_cast<const bf16x8 *>(lds + slot * Cfg::kKHalfBytes + koff[j][ks % kKSB] +
                                             (ks / kKSB) * 256);
  };
  // kCache: the PV operand from a key-major V tile by two transposing reads.
  // Within each 16 lanes, element e of lane i of such a read is element i & 3
  // at the address of lane 4 e + (i >> 2). So lane 16 q4 + 4 e + u points at
  // channels 16 cb + 4 u .. + 3 of key 32 kb + 8 q4 + 4 r + e (r: which 4-key
  // half), and lane 16 q4 + i receives keys 32 kb + 8 q4 + 4 r + 0..3 of
  // channel 16 cb + i. The key row's swizzle XORs the 32-byte unit index (cb
  // mod 8, mod 4 at d_h = 64) with swz_vc_unit of the key, which depends on
  // bits 0, 1, 3 of the key only: per-lane bases for cb mod 8, the rest
  // immediates.
  constexpr int kUnits = D >= 128 ? 8 : 4;  // 32-byte units per 256 bytes of a row
  constexpr int kTB = Cfg::kCB < kUnits ? Cfg::kCB : kUnits;
  int vtr[kTB];
  {
    const int e = (lane >> 2) & 3, u = lane & 3;
    const int key = 8 * q4 + e, f = swz_vc_unit<D>(key);
#pragma unroll
    for (int cl = 0; cl < kTB; ++cl)
      vtr[cl] = 4 * Cfg::kKHalfBytes + key * (2 * D) + 32 * (cl ^ f) + 8 * u;
  }
  auto vfrag = [&](int buf, int cb, int kb) {
    if constexpr (kCache) {
      typedef short s16x4 __attribute__((ext_vector_type(4)));
      typedef short s16x8 __attribute__((ext_vector_type(8)));
      char *p = lds + buf * Cfg::kVTileBytes + vtr[cb % kTB] + (cb / kTB) * 256 + 32 * kb * (2 * D);
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4 *)p);
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4 *)(p + 4 * (2 * D)));
      return __builtin_bit_cast(bf16x8, (s16x8)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    } else {
      return *reinterpret_cast<const bf16x8 *>(lds + buf * Cfg::kVTileBytes +
                                               cb * 16 * Cfg::kVRowBytes + voff[kb]);
    }
  };

  // Fixed softmax reference. The queries arrive scaled by log2(e), so a
  // logit x is already in base-2 units and p = exp2(x - U). |x| <= |q_t| |k_s|
  // (Cauchy-Schwarz) and a key after RMSNorm has |k| <= sqrt(d_h)
  // max_c |1 + gamma_k[c]|, so U_t = |q_t| sqrt(d_h) max|1 + gamma_k| bounds
  // every logit of row t: p <= 1 never overflows and there is no running max
  // or rescale of O. While 2 U_t <= 100 the row's largest p is >= 2^-100, far
  // from underflow; otherwise the workgroup first takes the exact row maxima
  // in a pass over its key tiles and uses those instead. Either way O and l
  // share the reference, which cancels in O / l. The S accumulators start at
  // -U_t, so the MFMAs deliver x - U_t directly.
  gmax = wave_max(gmax);
  float m_ref[kQB];
  float negu[kQB];  // -U_t (0 for a row without keys), the S accumulators' start
  auto neg_ref = [&](int qb) { return m_ref[qb] == -INFINITY ? 0.f : -m_ref[qb]; };
  // The start vector of an S accumulator, formed next to the MFMA that takes
  // it: the empty asm makes the value opaque, so the compiler writes the
  // copies where they are used instead of keeping them live through the loop.
  auto splat_ref = [&](int qb) {
    float u = negu[qb];
    asm volatile("" : "+v"(u));
    return f32x4{u, u, u, u};
  };
  // the 4 lanes holding the same query (q4 = 0..3) combine their partials
  auto quad_sum = [&](float x) {
    x += __shfl_xor(x, 16, kWave);
    return x + __shfl_xor(x, 32, kWave);
  };
  auto quad_max = [&](float x) {
    x = fmaxf(x, __shfl_xor(x, 16, kWave));
    return fmaxf(x, __shfl_xor(x, 32, kWave));
  };
  bool bound_ok = true;
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    float qq = 0.f;  // |q_t|^2: bf16 pairs squared and summed in fp32
#pragma unroll
    for (int ks = 0; ks < Cfg::kKS; ++ks)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x2 pr = {qf[qb][ks][2 * j], qf[qb][ks][2 * j + 1]};
        qq = __builtin_amdgcn_fdot2_f32_bf16(pr, pr, qq, false);
      }
    qq = quad_sum(qq);
    // 1% margin covers the bf16 rounding of the stored keys
    m_ref[qb] = sqrtf(qq) * sqrtf((float)D) * gmax * 1.01f;
    bound_ok = bound_ok && 2.f * m_ref[qb] <= 100.f;
    negu[qb] = neg_ref(qb);
  }
  // Zero reference: when U_t <= kZeroRefMax for every row of the wave, the
  // weights are taken as p = 2^x without any shift. They then lie in
  // [2^-kZeroRefMax, 2^kZeroRefMax] (|x| <= U_t), so neither p, l nor O can
  // overflow or lose their scale (O would need |V| > 2^(128 - kZeroRefMax - 17)
  // over 2^17 keys), and the S accumulators of the full tiles start from the
  // MFMA's inline zero instead of a per-row splat that costs four moves per
  // accumulator. The choice is per wave (every row of a wave takes the same
  // code path); the reference of its rows is 0 then, which the split-KV merge
  // sees in (m, l).
  constexpr float kZeroRefMax = 40.f;
  // d_h = 256 keeps a single copy of the tile loop: there the second copy
  // cost more in spilled registers than the moves it saves.
  constexpr bool kZeroRefCopy = D <= 128;
  bool zero_ok = (ref_flags & (kRefExactMax | kRefNoZero)) == 0;
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) zero_ok = zero_ok && m_ref[qb] <= kZeroRefMax;
  bool zero_ref = kZeroRefCopy && __all(zero_ok);

  // S of a 32-key half: 4 accumulators, quad qd = 2 qb + j (row block qb,
  // sub-tile j); lane element r of quad qd is key 8 q4 + 4 j + r of the half.
  using SHalf = f32x4[2 * kQB];
  // Which logits of a 32-key half starting at key s0 are allowed; blocked
  // ones become -inf. Allowed keys of a row form one interval; relative to
  // the lane's first key s0 + 8 q4, element r of sub-tile j sits at offset
  // e = 4 j + r, so one subtraction and one unsigned compare per element test
  // lo <= e <= hi: allowed(qb, e) = (unsigned)(e - lo[qb]) <= span[qb].
  struct HalfMask {
    int lo[kQB];
    uint32_t span[kQB];
    DEVI bool allowed(int qb, int e) const { return (uint32_t)(e - lo[qb]) <= span[qb]; }
  };
  auto mask_range = [&](int s0) {
    const int base = s0 + 8 * q4;
    HalfMask hm;
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      const int ta = a.q0 + my_t[qb];  // absolute index of the query
      int hi = min(ta, len - 1) - base;
      int lo = (a.local ? ta - a.window + 1 : -(1 << 30)) - base;
      if (hi < lo) {  // nothing allowed
        lo = 1 << 30;
        hi = lo;
      }
      hm.lo[qb] = lo;
      hm.span[qb] = (uint32_t)(hi - lo);
    }
    return hm;
  };
  auto qk_half = [&](int slot, SHalf &sv, bool from_ref) {
#pragma unroll
    for (int qd = 0; qd < 2 * kQB; ++qd) sv[qd] = from_ref ? splat_ref(qd >> 1) : f32x4{};
#pragma unroll
    for (int ks = 0; ks < Cfg::kKS; ++ks)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const bf16x8 kf = kfrag(slot, j, ks);
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb)
          sv[2 * qb + j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[qb][ks], sv[2 * qb + j], 0, 0, 0);
      }
  };

  // One step per 64-key tile it, as two 32-key halves (K halves u = 2 it and
  // 2 it + 1). While the softmax and PV of half u run, the S of half u + 1
  // goes to the matrix pipe. The work is a fixed sequence of groups of 4
  // fragments (one MFMA per row block for each fragment): for each
  // half, kNG groups of S MFMAs then kPG groups of PV MFMAs. The fragments of
  // group i + 1 are read from LDS while group i runs (across the halves; only
  // the tile's first group waits for its reads), each group carries its
  // share of the softmax arithmetic, and the first half issues the tile's
  // prefetches (K halves 2 it + 3, 2 it + 4 and V tile it + 1, into buffers
  // last read before the previous barrier), a few per group. A scheduling
  // fence closes each group: scheduled across groups, the 16x16x32 form held
  // more registers than the budget allows (spills at d_h = 128 and 256) and
  // ran slower. par_tag: the parity of `it` when known at compile time (then
  // every LDS slot and buffer index is an immediate), else -1.
  using Sc = TileSched<D, kQB>;
  constexpr int kG = Sc::kG, kNG = Sc::kNG, kNGT = Sc::kNGT, kPieces = Sc::kPieces, kPPG = Sc::kPPG;
  const bf16x2 ones = {(bf16)1.f, (bf16)1.f};

  auto tile_step = [&](auto masked_tag, auto next_tag, auto par_tag, auto zero_tag, int it,
                       SHalf &s_a, SHalf &s_b) {
    constexpr bool kMasked = decltype(masked_tag)::value;
    constexpr bool kZero = decltype(zero_tag)::value;  // S accumulators start at 0
    constexpr bool kNext = decltype(next_tag)::value;  // S of half 2 it + 2 is needed
    constexpr int kPar = decltype(par_tag)::value;
    const int par = kPar >= 0 ? kPar : (it & 1);
    const int s_tile = my_begin + it * kBN;

    // fragments of group gi of the tile (4 of them): S group gl, fragment j
    // is K sub-tile (4 gl + j) % 2 at k-step (4 gl + j) / 2; PV group gl,
    // fragment j is channel block 4 (gl - kNG) + j
    auto read_frags = [&](auto gi_tag, bf16x8 (&fr)[4]) {
      constexpr int gi = decltype(gi_tag)::value;
      constexpr int kb = gi / kNGT, gl = gi % kNGT;
      if constexpr (gl < kNG) {
        if constexpr (kb == 0 || kNext) {
#pragma unroll
          for (int j = 0; j < kG; ++j) {
            const int f = gl * kG + j;
            fr[j] = kfrag((2 * par + kb + 1) & 3, f & 1, f >> 1);
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < kG; ++j) fr[j] = vfrag(par, kG * (gl - kNG) + j, kb);
      }
    };
    auto issue_piece = [&](int pc) {
      if (pc < Cfg::kKHalfLoads)
        issue_k_piece(it + 1, 1, (2 * par + 3) & 3, pc);
      else if (pc < 2 * Cfg::kKHalfLoads)
        issue_k_piece(it + 2, 0, (2 * par) & 3, pc - Cfg::kKHalfLoads);
      else
        issue_v_piece(it + 1, par ^ 1, pc - 2 * Cfg::kKHalfLoads);
    };

    float ex[8 * kQB];
    bf16x8 pf[kQB];
    bf16x8 fr[4], frn[4];
    // masked tiles: allowed-logit bits of the current half (applied as the
    // exponentials read the S accumulators)
    HalfMask hm;
    if constexpr (kMasked) hm = mask_range(s_tile);
    read_frags(std::integral_constant<int, 0>{}, fr);
    static_for<2 * kNGT>([&](auto g_tag) {
      constexpr int gi = decltype(g_tag)::value;
      constexpr int kb = gi / kNGT, g = gi % kNGT;
      constexpr bool kS = g < kNG;
      constexpr bool kSActive = kS && (kb == 0 || kNext);
      SHalf &s_cur = kb == 0 ? s_a : s_b;
      SHalf &s_nxt = kb == 0 ? s_b : s_a;
      if constexpr (g == 0) {
        if constexpr (kb == 1 && kMasked) hm = mask_range(s_tile + 32);
      }
      if constexpr (gi + 1 < 2 * kNGT) read_frags(std::integral_constant<int, gi + 1>{}, frn);
      if constexpr (kSActive) {
#pragma unroll
        for (int j = 0; j < kG; ++j) {
          constexpr int f0 = g * kG;
          const int f = f0 + j, sj = f & 1, ks = f >> 1;
#pragma unroll
          for (int qb = 0; qb < kQB; ++qb)
            s_nxt[2 * qb + sj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                fr[j], qf[qb][ks],
                ks == 0 ? (kZero ? f32x4{} : splat_ref(qb)) : s_nxt[2 * qb + sj], 0, 0, 0);
        }
      } else if constexpr (!kS) {
#pragma unroll
        for (int j = 0; j < kG; ++j) {
          const int cb = kG * (g - kNG) + j;
#pragma unroll
          for (int qb = 0; qb < kQB; ++qb)
            acc_o[qb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fr[j], pf[qb], acc_o[qb][cb],
                                                                   0, 0, 0);
        }
      }
#pragma unroll
      for (int qd = 0; qd < 2 * kQB; ++qd) {
        if (Sc::e_grp(qd) == g) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float x = s_cur[qd][i];
            ex[4 * qd + i] =
                __builtin_amdgcn_exp2f(!kMasked || hm.allowed(qd >> 1, 4 * (qd & 1) + i) ? x
                                                                                 : -INFINITY);
          }
        }
        if (Sc::c_grp(qd) == g) {
#pragma unroll
          for (int i = 0; i < 4; ++i) pf[qd >> 1][4 * (qd & 1) + i] = (bf16)ex[4 * qd + i];
        }
        if (Sc::d_grp(qd) == g) {
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const bf16x2 pr = {pf[qd >> 1][4 * (qd & 1) + 2 * i],
                               pf[qd >> 1][4 * (qd & 1) + 2 * i + 1]};
            l_run[qd >> 1] = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, l_run[qd >> 1], false);
          }
        }
      }
      if constexpr (kb == 0) {
#pragma unroll
        for (int i = 0; i < kPPG; ++i)
          if (g * kPPG + i < kPieces) issue_piece(g * kPPG + i);
      }
      if constexpr (gi + 1 < 2 * kNGT) {
#pragma unroll
        for (int j = 0; j < 4; ++j) fr[j] = frn[j];
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    publish_tiles();  // this tile's prefetches have landed
  };

  // Tiles where no key is blocked for any row of the workgroup form one
  // range [it_lo, it_hi] (the conditions are monotone in the tile start);
  // they run a single straight-line body. The tiles before and after it (the
  // start of a sliding window, the causal diagonal, padding) and the last tile
  // take the masked body.
  int it_lo = 0, it_hi = -1;
  {
    const int hi_s0 = min(a.q0 + t_lo, len - 1) - (kBN - 1);  // s0 <= hi_s0
    const int lo_s0 = a.local ? a.q0 + t_hi - a.window : INT_MIN / 2;  // s0 >= lo_s0
    if (hi_s0 >= my_begin) it_hi = (hi_s0 - my_begin) / kBN;
    if (lo_s0 > my_begin) it_lo = div_up(lo_s0 - my_begin, kBN);
  }
  auto run = [&](auto zero_tag, SHalf &s_a) {
    using T_ = std::true_type;
    using F_ = std::false_type;
    SHalf s_b;
    using PR = std::integral_constant<int, -1>;
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    // Masked tiles always form the S of the next half (one code copy per
    // reference mode, fewer registers); after the last tile that reads a K
    // slot holding a clamped copy of the last tile, and the result is unused.
    auto masked_tile = [&](int it) { tile_step(T_{}, T_{}, PR{}, zero_tag, it, s_a, s_b); };
    auto full_tile = [&](auto par_tag, int it) {
      tile_step(F_{}, T_{}, par_tag, zero_tag, it, s_a, s_b);
    };
    const int head_end = min(it_lo, n_tiles);
    const int full_end = min(it_hi + 1, n_tiles - 1);
    // One masked loop (one copy of its code): the head segment, then the full
    // tiles in pairs of known parity, then the tail segment.
    int it = 0;
#pragma nounroll
    for (int seg = 0; seg < 2; ++seg) {
      const int seg_end = seg == 0 ? head_end : n_tiles;
      for (; it < seg_end; ++it) masked_tile(it);
      if (seg == 0) {
        if (it < full_end && (it & 1)) full_tile(P1{}, it++);
        for (; it + 1 < full_end; it += 2) {
          full_tile(P0{}, it);
          full_tile(P1{}, it + 1);
        }
        if (it < full_end) full_tile(P0{}, it++);
      }
    }
  };
  // S of K half 0; the barrier after it orders these reads before any later
  // write to slot 0
  SHalf s0_first;
  if (n_tiles > 0) {
    qk_half(0, s0_first, !zero_ref);
  } else {
#pragma unroll
    for (int qd = 0; qd < 2 * kQB; ++qd) s0_first[qd] = f32x4{};
  }
  if (!__syncthreads_and(bound_ok) || (ref_flags & kRefExactMax)) {
    // Exact row maxima (log2 units) over the allowed keys: each tile's two K
    // halves go to slots 0 and 1, S MFMAs only. Rare; kept simple.
    float mx[kQB];
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) mx[qb] = -INFINITY;
    for (int it = 0; it < n_tiles; ++it) {
#pragma unroll
      for (int kbh = 0; kbh < 2; ++kbh)
#pragma unroll
        for (int i = 0; i < Cfg::kKHalfLoads; ++i) issue_k_piece(it, kbh, kbh, i);
      publish_tiles();
#pragma unroll
      for (int kbh = 0; kbh < 2; ++kbh) {
        SHalf sv;
        qk_half(kbh, sv, false);
        const HalfMask hk = mask_range(my_begin + it * kBN + 32 * kbh);
#pragma unroll
        for (int qd = 0; qd < 2 * kQB; ++qd)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            mx[qd >> 1] = fmaxf(mx[qd >> 1],
                                hk.allowed(qd >> 1, 4 * (qd & 1) + r) ? sv[qd][r] : -INFINITY);
      }
      __syncthreads();  // reads done before the next tile overwrites the slots
    }
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      m_ref[qb] = quad_max(mx[qb]);
      negu[qb] = neg_ref(qb);
    }
    zero_ref = false;
    issue_prologue();
    publish_tiles();
    if (n_tiles > 0) qk_half(0, s0_first, true);
    __syncthreads();
  }
  bool ran = false;
  if constexpr (kZeroRefCopy) {
    if (zero_ref) {
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb) m_ref[qb] = 0.f;
      run(std::true_type{}, s0_first);
      ran = true;
    }
  }
  if (!ran) run(std::false_type{}, s0_first);

  // Normalise. Several chunks: each lane stores its fp32 partial output (4
  // channels 16 cb + 4 q4 + [0, 4) of row 16 qb + qc per accumulator) and the
  // row's (m, l) straight from registers; the merge reads them at full
  // precision. A single chunk writes the bf16 output rows: the K/V buffers are
  // free after the last tile's barrier, so each wave stages its 16 kQB rows (a
  // 16-byte pad per row) in a region of its own, then writes them back as
  // whole rows of 16-byte pieces.
  if (geo.n_active > 1) {  // uniform per block
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      const float l_tot = quad_sum(l_run[qb]);
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      if (my_t[qb] >= a.T) continue;
      const size_t row = (((size_t)split * a.B + b) * a.H + h) * a.T + my_t[qb];
#pragma unroll
      for (int cb = 0; cb < Cfg::kCB; ++cb)
        *reinterpret_cast<f32x4 *>(part_o + row * D + 16 * cb + 4 * q4) = acc_o[qb][cb] * inv;
      if (q4 == 0) {
        part_ml[2 * row] = m_ref[qb];
        part_ml[2 * row + 1] = l_tot;
      }
    }
    return;
  }
  constexpr int kPitch = 2 * D + 16;
  static_assert(4 * kRPW * kPitch <= Cfg::kLdsBytes, "output staging fits the tile buffers");
  char *stage = lds + w * kRPW * kPitch;
  constexpr int kPieces16 = D / 8;  // 16-byte pieces per row
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    const float l_tot = quad_sum(l_run[qb]);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
    for (int cb = 0; cb < Cfg::kCB; ++cb) {
      bf16x4 v;
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = (bf16)(acc_o[qb][cb][r] * inv);
      *reinterpret_cast<bf16x4 *>(stage + (16 * qb + qc) * kPitch + 2 * (16 * cb + 4 * q4)) = v;
    }
  }
  // the same wave reads its region back (LDS keeps a wave's accesses in order)
#pragma unroll
  for (int i = 0; i < kRPW * kPieces16 / kWave; ++i) {
    const int item = i * kWave + lane;
    const int r = item / kPieces16, c = item % kPieces16;
    const int t = wq0 + r;
    const u32x4 v = *reinterpret_cast<const u32x4 *>(stage + r * kPitch + 16 * c);
    if (t >= a.T) continue;
    bf16 *dst = o + ((size_t)b * a.T + t) * ((size_t)a.H * D) + (size_t)h * D;
    *reinterpret_cast<u32x4 *>(dst + 8 * c) = v;
  }
}

// Merge the key chunks of query tiles that had more than one:
// o = sum_j 2^(m_j - M) l_j o_j / sum_j 2^(m_j - M) l_j. kCombineSlices
// workgroups per query tile (blockIdx.x in the attention kernel's base
// order); tiles with a single chunk were written by the attention kernel and
// exit at once. A thread handles 8 channels of a row per item: every chunk's
// 32 bytes of fp32 partial output and (m, l) pair of the item are loaded
// before any arithmetic, several items at a time (one round trip per batch).
constexpr int kCombineItems = 2;   // items in flight per thread
constexpr int kCombineSlices = 8;  // workgroups per query tile

template <int D>
__global__ void __launch_bounds__(256)
flash_combine(const int32_t *__restrict__ kv_len, bf16 *__restrict__ o,
              const float *__restrict__ part_o, const float *__restrict__ part_ml, AttnArgs a,
              int gp, int n_qtiles, int n_hgrp, int n_split, int chunk_keys, int rpw) {
  const Geo geo = geometry(a, kv_len, blockIdx.x, gp, n_qtiles, n_hgrp, chunk_keys, rpw);
  if (geo.n_active <= 1) return;  // uniform per block
  constexpr int kC8 = D / 8;  // 8-channel pieces per row
  const int G = a.H / a.Hk;
  const int h0 = geo.kh * G + geo.hgrp * gp;
  const int nt = geo.t_hi - geo.t_lo;
  const int n_items = gp * nt * kC8;
  const int na = geo.n_active;
  for (int base = blockIdx.y * 256 + threadIdx.x; base < n_items;
       base += 256 * kCombineSlices * kCombineItems) {
    float w[kCombineItems][8], lw[kCombineItems][8];
    f32x4 v[kCombineItems][8][2];
#pragma unroll
    for (int u = 0; u < kCombineItems; ++u) {
      const int item = base + 256 * kCombineSlices * u;
      const bool ok = item < n_items;
      const int c8 = item % kC8, r = item / kC8;
      const int h = h0 + r / nt, t = geo.t_lo + r % nt;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        w[u][j] = -INFINITY;
        lw[u][j] = 0.f;
        v[u][j][0] = v[u][j][1] = f32x4{};
        if (ok && j < na) {
          const size_t row = (((size_t)j * a.B + geo.b) * a.H + h) * a.T + t;
          const float2 ml = *reinterpret_cast<const float2 *>(part_ml + 2 * row);
          w[u][j] = ml.x;  // m_j
          lw[u][j] = ml.y; // l_j
#pragma unroll
          for (int e = 0; e < 2; ++e)
            v[u][j][e] = *reinterpret_cast<const f32x4 *>(part_o + row * D + 8 * c8 + 4 * e);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kCombineItems; ++u) {
      const int item = base + 256 * kCombineSlices * u;
      if (item >= n_items) break;
      const int c8 = item % kC8, r = item / kC8;
      const int h = h0 + r / nt, t = geo.t_lo + r % nt;
      float M = -INFINITY;
#pragma unroll
      for (int j = 0; j < 8; ++j) M = fmaxf(M, w[u][j]);
      const float mu = M == -INFINITY ? 0.f : M;
      float num[8] = {}, den = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j >= na) break;
        const float wl = exp2f(w[u][j] - mu) * lw[u][j];
        den += wl;
#pragma unroll
        for (int i = 0; i < 8; ++i) num[i] = fmaf(wl, v[u][j][i >> 2][i & 3], num[i]);
      }
      bf16x8 out;
#pragma unroll
      for (int i = 0; i < 8; ++i) out[i] = (bf16)(den > 0.f ? num[i] / den : 0.f);
      *reinterpret_cast<bf16x8 *>(o + ((size_t)geo.b * a.T + t) * ((size_t)a.H * D) +
                                  (size_t)h * D + 8 * c8) = out;
    }
  }
}

struct Plan {
  int qb, gp, n_qtiles, n_hgrp, n_split, chunk_keys, remap;
  long n_base;
};

// Planning constants (units: one 64-key tile of one workgroup, about 1.8 us
// on the 1B shape). A workgroup's prologue (Q, first K/V tiles, reference)
// costs about 2.5 tiles; a split adds the merge launch and its reads, about
// 8 (measured: splitting the 1B-shaped local layer in two is slower).
constexpr double kPrologueTiles = 2.5, kMergeTiles = 8.0;
constexpr int kCUs = 256;  // MI355X compute units
// workgroups resident per CU: two at d_h <= 128 (64 KB of LDS and at most
// 256 registers per lane each), one at d_h = 256 (131 KB, 512 registers)
constexpr int wgs_per_cu(int d_h) { return d_h <= 128 ? 2 : 1; }

Plan plan_qb(const AttnArgs &a, int qb) {
  Plan p;
  p.qb = qb;
  const int G = a.H / a.Hk;
  p.gp = (G % 4 == 0) ? 4 : (G % 2 == 0) ? 2 : 1;
  // (a window covering every key takes the global layer's plan and bits)
  const int slots = kCUs * wgs_per_cu(a.d_h);  // workgroups running at once
  const int TQ = 16 * qb * (4 / p.gp);
  p.n_qtiles = div_up_h(a.T, TQ);
  p.n_hgrp = G / p.gp;
  const long n_groups = (long)a.B * a.Hk * p.n_hgrp;
  p.n_base = n_groups * p.n_qtiles;
  // XCD-contiguous order when whole (b, kh, head group) runs divide evenly
  // among the 8 XCDs (each L2 then holds the K/V its CUs share), and on
  // sliding-window layers (every query tile spans about W keys, so runs of
  // neighbouring tiles stay balanced and share most of their window in one
  // L2; measured: the 1B-shaped local layer's time unchanged, its K/V read
  // by one XCD each instead of all eight); otherwise the plain order, which
  // deals neighbouring causal query tiles to different XCDs and keeps their
  // loads balanced.
  p.remap = n_groups % 8 == 0 || a.local;
  // Key tiles of query tile qt (data-independent: padding is ignored here).
  auto tiles_of = [&](int qt) {
    const int t_lo = qt * TQ, t_hi = min(a.T, t_lo + TQ);
    const int kv_begin = a.local ? max(0, a.q0 + t_lo - a.window + 1) : 0;
    return div_up_h(a.q0 + t_hi - (kv_begin / kBN) * kBN, kBN);
  };
  int max_tiles = 0;
  for (int qt = 0; qt < p.n_qtiles; ++qt) max_tiles = max(max_tiles, tiles_of(qt));
  // Split key ranges only when the query tiles alone leave CUs idle: pick
  // the chunk count minimising rounds x (chunk + prologue) (+ merge), where
  // a round is `slots` concurrent workgroups of similar length.
  p.n_split = 1;
  if (p.n_base < slots) {
    double best = max_tiles + kPrologueTiles;
    for (int ns = 2; ns <= 8; ++ns) {  // flash_combine merges at most 8 chunks
      const int c = div_up_h(max_tiles, ns);
      long active = 0;
      for (int qt = 0; qt < p.n_qtiles; ++qt) active += div_up_h(tiles_of(qt), c);
      active *= n_groups;
      const double cost = div_up_h(active, slots) * (c + kPrologueTiles) + kMergeTiles;
      if (cost < best) {
        best = cost;
        p.n_split = ns;
      }
    }
  }
  // one chunk covers every key range when there is no split
  p.chunk_keys = p.n_split == 1 ? a.q0 + a.T + kBN : div_up_h(max_tiles, p.n_split) * kBN;
  return p;
}

// One row block per wave (twice the workgroups, each with half the rows)
// where two blocks leave at least half the chip idle on a sliding-window layer
// at d_h = 256 (one workgroup per CU): its query tiles all take about the
// same number of keys, so the doubled grid fills the CUs in one round.
// Measured on the 1B-shaped local layer: 25.5 -> 20.3 us. On causal global
// layers of that size the split plan with two blocks stays faster (61
// against 72 us unsplit with one block).
Plan plan(const AttnArgs &a) {
  const Plan p2 = plan_qb(a, 2);
  if (a.local && a.d_h == 256 && 2 * p2.n_base <= (long)kCUs * wgs_per_cu(a.d_h))
    return plan_qb(a, 1);
  return p2;
}

template <int D, bool kCache, int kQB>
hipError_t launch_kernels(const bf16 *q, const bf16 *k, const bf16 *vt, const int32_t *kv_len,
                     const bf16 *gamma_k, bf16 *o, float *part_o, float *part_ml,
                     const AttnArgs &a, const Plan &p, int ref_flags, hipStream_t s) {
  using Cfg = AttnCfg<D>;
  auto kern = flash_attn_fwd_bf16<D, kCache, kQB>;
  hipError_t e = hipFuncSetAttribute((const void *)kern,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, Cfg::kLdsBytes);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)(p.n_base * p.n_split)),
                     dim3(kThreads), Cfg::kLdsBytes, s, q, k, vt, kv_len, gamma_k, o, part_o,
                     part_ml, a, p.gp, p.n_qtiles, p.n_hgrp, p.n_split, p.chunk_keys, p.remap,
                     ref_flags);
  e = hipGetLastError();
  if (e != hipSuccess || p.n_split == 1) return e;
  hipLaunchKernelGGL(flash_combine<D>, dim3((unsigned)p.n_base, kCombineSlices), dim3(256), 0, s,
                     kv_len,
                     o, part_o, part_ml, a, p.gp, p.n_qtiles, p.n_hgrp, p.n_split, p.chunk_keys,
                     16 * kQB);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const bf16 *q, const bf16 *k, const bf16 *vt, const int32_t *kv_len,
                    const bf16 *gamma_k, bf16 *o, float *part_o, float *part_ml, const AttnArgs &a,
                    int ref_flags, hipStream_t s) {
  const Plan p = plan(a);
  if constexpr (D == 256) {
    if (p.qb == 1)
      return a.S_cache > 0 ? launch_kernels<D, true, 1>(q, k, vt, kv_len, gamma_k, o, part_o,
                                                        part_ml, a, p, ref_flags, s)
                           : launch_kernels<D, false, 1>(q, k, vt, kv_len, gamma_k, o, part_o,
                                                         part_ml, a, p, ref_flags, s);
  }
  return a.S_cache > 0 ? launch_kernels<D, true, 2>(q, k, vt, kv_len, gamma_k, o, part_o,
                                                    part_ml, a, p, ref_flags, s)
                       : launch_kernels<D, false, 2>(q, k, vt, kv_len, gamma_k, o, part_o,
                                                     part_ml, a, p, ref_flags, s);
}

}  // namespace

size_t flash_attn_partial_bytes(const AttnArgs &a) {
  const Plan p = plan(a);
  if (p.n_split == 1) return 0;
  return (size_t)p.n_split * a.B * a.H * a.T * ((size_t)a.d_h * 4 + 8);
}

size_t flash_attn_partial_bytes_bound(const AttnArgs &a) {
  // key ranges are split (into at most 8 chunks) only when the query tiles
  // alone leave CUs idle, and that count does not depend on q0
  if (plan_qb(a, 2).n_base >= (long)kCUs * wgs_per_cu(a.d_h)) return 0;
  return (size_t)8 * a.B * a.H * a.T * ((size_t)a.d_h * 4 + 8);
}

hipError_t launch_flash_attn_bf16(const bf16 *q, const bf16 *k, const bf16 *vt,
                                  const int32_t *kv_len, const bf16 *gamma_k, bf16 *o,
                                  void *partial, const AttnArgs &a, int ref_flags,
                                  hipStream_t s) {
  const size_t rows = (size_t)plan(a).n_split * a.B * a.H * a.T;
  float *part_o = (float *)partial;
  float *part_ml = partial ? (float *)((char *)partial + rows * a.d_h * 4) : nullptr;
  switch (a.d_h) {
    case 64: return launch_d<64>(q, k, vt, kv_len, gamma_k, o, part_o, part_ml, a, ref_flags, s);
    case 128: return launch_d<128>(q, k, vt, kv_len, gamma_k, o, part_o, part_ml, a, ref_flags, s);
    case 256: return launch_d<256>(q, k, vt, kv_len, gamma_k, o, part_o, part_ml, a, ref_flags, s);
    default: return hipErrorInvalidValue;
  }
}
