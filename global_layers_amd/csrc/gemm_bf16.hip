// bf16 projections on gfx950 MFMA ("Gemma 3 Attention Block", How it works:
// q_einsum / kv_einsum produce Q, K, V from x; attn_vec_einsum maps the heads
// back to D). Both are C[M,N] = A[M,K] * B[N,K]^T with A the activations and
// B an output-major weight, accumulated in fp32.
//
//  * gemm_bf16_nt: prefill. Block tile BM x BN x 64, waves arranged WM x WN,
//    32x32x16 bf16 MFMAs, LDS double buffer fed through registers so the next
//    K slice's global loads overlap the current slice's MFMAs. The MFMA is
//    issued with the weight fragment as its first operand so that each lane
//    ends up holding 4 consecutive output columns (one 8-byte store).
//  * gemv16_bf16_splitk: decode (M = batch <= 16 per M block). Weight-streaming
//    16x16x32 MFMAs, each wave one 16-column block over one K split, fp32
//    partials per split; the consumer adds the splits.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int kBK = 64;
constexpr int kPad = 8;                // bf16 elements of row padding in LDS
constexpr int kLdsRow = kBK + kPad;    // 72 elements = 144 bytes

template <int BM, int BN, int WM, int WN>
struct GemmCfg {
  static constexpr int kThreads = WM * WN * kWave;
  static constexpr int kWaveM = BM / WM, kWaveN = BN / WN;
  static constexpr int kFM = kWaveM / 32, kFN = kWaveN / 32;
  static constexpr int kChunksA = BM * kBK / 8 / kThreads;  // 16-byte chunks per thread
  static constexpr int kChunksB = BN * kBK / 8 / kThreads;
  static constexpr int kLdsElems = 2 * (BM + BN) * kLdsRow;
  static_assert(kWaveM % 32 == 0 && kWaveN % 32 == 0, "wave tile must be 32-aligned");
  static_assert(BM * kBK / 8 % kThreads == 0 && BN * kBK / 8 % kThreads == 0, "chunking");
};

template <int BM, int BN, int WM, int WN>
__global__ void __launch_bounds__(WM * WN * 64)
gemm_bf16_nt(const bf16 *__restrict__ A, const bf16 *__restrict__ B0, const bf16 *__restrict__ B1,
             int N0, bf16 *__restrict__ C, int M, int N, int K, int n_tiles_n) {
  using Cfg = GemmCfg<BM, BN, WM, WN>;
  extern __shared__ __attribute__((aligned(16))) bf16 lds[];
  bf16 *As = lds;                       // [2][BM][kLdsRow]
  bf16 *Bs = lds + 2 * BM * kLdsRow;    // [2][BN][kLdsRow]

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int n_blocks = gridDim.x;
  const int bid = xcd_remap(blockIdx.x, n_blocks);
  // tiles of one row of C (same A rows) stay adjacent in the logical order
  const int tile_m = bid / n_tiles_n, tile_n = bid % n_tiles_n;
  const int m0 = tile_m * BM, n0 = tile_n * BN;

  u32x4 ra[Cfg::kChunksA], rb[Cfg::kChunksB];
  auto load_global = [&](int k0) {
#pragma unroll
    for (int i = 0; i < Cfg::kChunksA; ++i) {
      const int c = tid + i * Cfg::kThreads;
      const int r = c / (kBK / 8), kc = (c % (kBK / 8)) * 8;
      const int gm = m0 + r;
      ra[i] = gm < M ? ld16(A + (size_t)gm * K + k0 + kc) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < Cfg::kChunksB; ++i) {
      const int c = tid + i * Cfg::kThreads;
      const int r = c / (kBK / 8), kc = (c % (kBK / 8)) * 8;
      const int gn = n0 + r;
      const bf16 *src = gn < N0 ? B0 + (size_t)gn * K : B1 + (size_t)(gn - N0) * K;
      rb[i] = gn < N ? ld16(src + k0 + kc) : u32x4{0, 0, 0, 0};
    }
  };
  auto store_lds = [&](int buf) {
    bf16 *as = As + buf * BM * kLdsRow, *bs = Bs + buf * BN * kLdsRow;
#pragma unroll
    for (int i = 0; i < Cfg::kChunksA; ++i) {
      const int c = tid + i * Cfg::kThreads;
      st16(as + (c / (kBK / 8)) * kLdsRow + (c % (kBK / 8)) * 8, ra[i]);
    }
#pragma unroll
    for (int i = 0; i < Cfg::kChunksB; ++i) {
      const int c = tid + i * Cfg::kThreads;
      st16(bs + (c / (kBK / 8)) * kLdsRow + (c % (kBK / 8)) * 8, rb[i]);
    }
  };

  f32x16 acc[Cfg::kFM][Cfg::kFN];
#pragma unroll
  for (int i = 0; i < Cfg::kFM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::kFN; ++j) acc[i][j] = f32x16{};

  const int nk = K / kBK;
  load_global(0);
  store_lds(0);
  __syncthreads();

  const int lrow = lane & 31, lk = (lane >> 5) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_global((kt + 1) * kBK);
    const bf16 *as = As + buf * BM * kLdsRow + (wm * Cfg::kWaveM + lrow) * kLdsRow + lk;
    const bf16 *bs = Bs + buf * BN * kLdsRow + (wn * Cfg::kWaveN + lrow) * kLdsRow + lk;
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      bf16x8 af[Cfg::kFM], bfr[Cfg::kFN];
#pragma unroll
      for (int i = 0; i < Cfg::kFM; ++i)
        af[i] = *reinterpret_cast<const bf16x8 *>(as + i * 32 * kLdsRow + kk * 16);
#pragma unroll
      for (int j = 0; j < Cfg::kFN; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8 *>(bs + j * 32 * kLdsRow + kk * 16);
#pragma unroll
      for (int i = 0; i < Cfg::kFM; ++i)
#pragma unroll
        for (int j = 0; j < Cfg::kFN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store_lds(buf ^ 1);
    __syncthreads();
  }

  // acc[i][j] holds D[n][m]: lane column m = lane % 32, rows n = 8g + 4h + r.
  const int h = lane >> 5;
#pragma unroll
  for (int i = 0; i < Cfg::kFM; ++i) {
    const int gm = m0 + wm * Cfg::kWaveM + i * 32 + lrow;
    if (gm >= M) continue;
#pragma unroll
    for (int j = 0; j < Cfg::kFN; ++j) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int gn = n0 + wn * Cfg::kWaveN + j * 32 + 8 * g + 4 * h;
        bf16x4 v;
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = (bf16)acc[i][j][g * 4 + r];
        if (gn + 3 < N) {
          *reinterpret_cast<bf16x4 *>(C + (size_t)gm * N + gn) = v;
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (gn + r < N) C[(size_t)gm * N + gn + r] = v[r];
        }
      }
    }
  }
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_gemm(const bf16 *A, const bf16 *B0, const bf16 *B1, int N0, bf16 *C, int M,
                       int N, int K, hipStream_t s) {
  using Cfg = GemmCfg<BM, BN, WM, WN>;
  const int tm = div_up_h(M, BM), tn = div_up_h(N, BN);
  const size_t lds = Cfg::kLdsElems * sizeof(bf16);
  hipError_t e = hipFuncSetAttribute((const void *)gemm_bf16_nt<BM, BN, WM, WN>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((gemm_bf16_nt<BM, BN, WM, WN>), dim3(tm * tn), dim3(Cfg::kThreads), lds, s,
                     A, B0, B1, N0, C, M, N, K, tn);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Decode projections: P[split][m][n] = sum_{k in split} A[m][k] * W[n][k]
// ---------------------------------------------------------------------------
constexpr int kGemvWaves = 4;
constexpr int kGemvUnroll = 4;

__global__ void __launch_bounds__(kGemvWaves * 64)
gemv16_bf16_splitk(const bf16 *__restrict__ A, const bf16 *__restrict__ W0,
                   const bf16 *__restrict__ W1, int N0, float *__restrict__ P, int M, int N, int K,
                   int k_per_split) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nb = blockIdx.x * kGemvWaves + wave;       // 16-column block
  const int split = blockIdx.y, mb = blockIdx.z;
  if (nb * 16 >= N) return;
  const int n = nb * 16 + (lane & 15);
  const int m = mb * 16 + (lane & 15);
  const int koff = (lane >> 4) * 8;
  const int k_begin = split * k_per_split, k_end = k_begin + k_per_split;
  const bool n_ok = n < N, m_ok = m < M;
  const int nn = n_ok ? n : 0;
  const bf16 *wp = (nn < N0 ? W0 + (size_t)nn * K : W1 + (size_t)(nn - N0) * K) + koff;
  const bf16 *ap = A + (size_t)(m_ok ? m : 0) * K + koff;

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  int k = k_begin;
  for (; k + 32 * kGemvUnroll <= k_end; k += 32 * kGemvUnroll) {
    u32x4 wv[kGemvUnroll], av[kGemvUnroll];
#pragma unroll
    for (int u = 0; u < kGemvUnroll; ++u) {
      wv[u] = ld16(wp + k + u * 32);
      av[u] = ld16(ap + k + u * 32);
    }
#pragma unroll
    for (int u = 0; u < kGemvUnroll; ++u) {
      if (!n_ok) wv[u] = u32x4{0, 0, 0, 0};
      if (!m_ok) av[u] = u32x4{0, 0, 0, 0};
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av[u]),
                                                     __builtin_bit_cast(bf16x8, wv[u]), acc,
                                                     0, 0, 0);
    }
  }
  for (; k < k_end; k += 32) {
    u32x4 wv = n_ok ? ld16(wp + k) : u32x4{0, 0, 0, 0};
    u32x4 av = m_ok ? ld16(ap + k) : u32x4{0, 0, 0, 0};
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                   __builtin_bit_cast(bf16x8, wv), acc, 0, 0, 0);
  }
  // D[m][n]: lane column n = lane % 16, rows m = (lane / 16) * 4 + r.
  const int col = nb * 16 + (lane & 15);
  if (col >= N) return;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = mb * 16 + (lane >> 4) * 4 + r;
    if (row < M) P[((size_t)split * M + row) * N + col] = acc[r];
  }
}

}  // namespace

hipError_t launch_gemm_bf16_nt(const bf16 *A, const bf16 *B0, const bf16 *B1, int N0, bf16 *C,
                               int M, int N, int K, hipStream_t s) {
  // Big problems: 256x256 tiles (8 waves, 2 per SIMD). Smaller ones: 128x128
  // tiles so that the grid still covers the 256 CUs.
  const long tiles256 = (long)div_up_h(M, 256) * div_up_h(N, 256);
  if (tiles256 >= 512) return launch_gemm<256, 256, 2, 4>(A, B0, B1, N0, C, M, N, K, s);
  return launch_gemm<128, 128, 2, 2>(A, B0, B1, N0, C, M, N, K, s);
}

int gemv_ksplit(int N, int K) {
  const int nblk = div_up_h(N, 16);
  int s = 1;
  while (s < 16 && (long)nblk * s < 2048) s *= 2;
  while (s > 1 && (K / 32) % s != 0) s /= 2;
  return s;
}

hipError_t launch_gemv16_bf16(const bf16 *A, const bf16 *W0, const bf16 *W1, int N0, float *P,
                              int M, int N, int K, int ksplit, hipStream_t s) {
  dim3 grid(div_up_h(div_up_h(N, 16), kGemvWaves), ksplit, div_up_h(M, 16));
  hipLaunchKernelGGL(gemv16_bf16_splitk, grid, dim3(kGemvWaves * 64), 0, s, A, W0, W1, N0, P, M,
                     N, K, K / ksplit);
  return hipGetLastError();
}
