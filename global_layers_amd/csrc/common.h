// Shared device helpers for the gfx950 attention kernels: element types,
// MFMA operand vectors, bf16 conversion and wave-level reductions.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>
#include <stdint.h>

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define DEVI __device__ __forceinline__

constexpr int kWave = 64;

DEVI float to_f32(float v) { return v; }
DEVI float to_f32(bf16 v) { return (float)v; }

template <typename T> DEVI T from_f32(float v);
template <> DEVI float from_f32<float>(float v) { return v; }
template <> DEVI bf16 from_f32<bf16>(float v) { return (bf16)v; }  // round to nearest even

// 16-byte vector load/store helpers (addresses must be 16-byte aligned).
DEVI u32x4 ld16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }
DEVI void st16(void *p, u32x4 v) { *reinterpret_cast<u32x4 *>(p) = v; }

DEVI float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

DEVI float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// Sum over aligned groups of `n` lanes (n a power of two <= 64).
template <int n> DEVI float group_sum(float v) {
#pragma unroll
  for (int o = n / 2; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Sum over aligned groups of n <= 16 lanes with DPP lane moves (no LDS
// round trip): neighbour swap, pair swap, then mirrors inside 8 and 16 lanes.
// Every step adds two operands in either order, so all lanes of a group end
// with the same bits.
template <int n> DEVI float group_sum_dpp(float v) {
  static_assert(n == 1 || n == 2 || n == 4 || n == 8 || n == 16, "group of at most 16 lanes");
  auto mv = [](float x, auto ctrl) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), decltype(ctrl)::value, 0xF,
                                        0xF, true));
  };
  if constexpr (n >= 2) v += mv(v, std::integral_constant<int, 0xB1>{});   // quad_perm 1,0,3,2
  if constexpr (n >= 4) v += mv(v, std::integral_constant<int, 0x4E>{});   // quad_perm 2,3,0,1
  if constexpr (n >= 8) v += mv(v, std::integral_constant<int, 0x141>{});  // row_half_mirror
  if constexpr (n >= 16) v += mv(v, std::integral_constant<int, 0x140>{}); // row_mirror
  return v;
}

DEVI int div_up(int a, int b) { return (a + b - 1) / b; }

// Remap a linear block id so that runs of consecutive logical ids land on the
// same XCD: the dispatcher deals workgroups round-robin over the 8 XCDs, so
// physical id p runs on XCD p % 8. Ids past the largest multiple of 8 keep
// their own value.
DEVI int xcd_remap(int p, int n) {
  const int full = n & ~7;
  if (p >= full) return p;
  const int per = full >> 3;
  return (p & 7) * per + (p >> 3);
}

constexpr float kLog2e = 1.4426950408889634f;

// s_waitcnt immediate (gfx9 encoding) that waits for vmcnt == 0 and leaves the
// expcnt and lgkmcnt counters unconstrained.
constexpr int kWaitVmcnt0 = (0x7 << 4) | (0xF << 8);

// One direct global -> LDS load (gfx950 global_load_lds_dwordx4): lane l
// moves the 16 bytes at sbase + lane_off (sbase wave-uniform) to LDS byte
// lds_wave_off + 16 l (lds_wave_off wave-uniform). The LDS destination goes
// in M0, bound as an input operand so the compiler sets M0 itself and knows
// it is taken. Inline assembly rather than the builtin: the compiler would
// count an LDS-writing load as a memory access of unknown order and make
// every later LDS fragment read wait for all LDS reads in flight; hidden from
// it, those reads keep their partial waits (which stay correct whether or not
// the load also counts in lgkmcnt: waiting for <= k outstanding still retires
// the oldest reads). Callers therefore wait for completion explicitly (vmcnt)
// before the barrier that hands the data to other waves, and only ever target
// a buffer that no wave reads before that barrier.
DEVI void load_lds16(const void *sbase, uint32_t lane_off, uint32_t lds_wave_off) {
  asm volatile("global_load_lds_dwordx4 %0, %1"
               :
               : "v"(lane_off), "s"(sbase), "{m0}"(lds_wave_off)
               : "memory");
}

// GeGLU activation of one element pair ("Full Gemma 3 Block", How it works:
// the MLP's GELU, tanh approximation, times the up projection), in fp32.
// Shared by the stand-alone activation pass and the gate|up projection's
// fused epilogue, so both round the same value.
DEVI float gelu_tanh_times(float x, float u) {
  const float t = tanhf(0.7978845608028654f * fmaf(0.044715f * x * x, x, x));
  return 0.5f * x * (1.f + t) * u;
}

// RoPE rotation of one channel pair at integer position p: angle
// p / scale * inv_freq, reduced modulo one turn in fp64 (positions reach
// 131071, where an fp32 angle would be off by ~1e-2 rad), then fp32 sincos.
DEVI void rope_sincos(int p, double inv_scale, double inv_freq, float &c, float &s) {
  const double two_pi = 6.283185307179586476925286766559;
  double a = (double)p * inv_scale * inv_freq;
  a -= rint(a * (1.0 / two_pi)) * two_pi;
  sincosf((float)a, &s, &c);
}
