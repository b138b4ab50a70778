// Device-side helpers shared by the MoE kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_internal.h"

namespace moe {

constexpr int kWave = 64;

typedef uint16_t bf16_t;           // raw bfloat16 bits
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest bfloat16, ties to even (inputs are finite).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// Eight consecutive elements as float: one 16-byte vector (bf16) or two (float).
template <typename T>
struct vec8;  // eight elements as one or two 16-byte vectors
template <>
struct vec8<bf16_t> {
  static __device__ __forceinline__ void load(const bf16_t* p, float* v) {
    const u32x4 r = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(r[i] << 16);
      v[2 * i + 1] = __uint_as_float(r[i] & 0xFFFF0000u);
    }
  }
  static __device__ __forceinline__ void store(bf16_t* p, const float* v) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
    *reinterpret_cast<u32x4*>(p) = r;
  }
};
template <>
struct vec8<float> {
  static __device__ __forceinline__ void load(const float* p, float* v) {
    const floatx4 a = *reinterpret_cast<const floatx4*>(p);
    const floatx4 b = *reinterpret_cast<const floatx4*>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = a[i];
      v[4 + i] = b[i];
    }
  }
  static __device__ __forceinline__ void store(float* p, const float* v) {
    *reinterpret_cast<floatx4*>(p) = floatx4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<floatx4*>(p + 4) = floatx4{v[4], v[5], v[6], v[7]};
  }
};

// Element access for the two storage types.
template <typename T> struct elem;
template <> struct elem<float> {
  __device__ static float load(const float* p) { return *p; }
  __device__ static float to_f32(float v) { return v; }
  __device__ static float from_f32(float v) { return v; }
};
template <> struct elem<bf16_t> {
  __device__ static float to_f32(bf16_t v) { return bf16_to_f32(v); }
  __device__ static bf16_t from_f32(float v) { return f32_to_bf16(v); }
};

__device__ __forceinline__ float act_relu(float z) { return z > 0.f ? z : 0.f; }

// GELU with the Gaussian CDF, z * Phi(z).  Phi comes from the complementary
// error function in the form of Abramowitz & Stegun, Handbook of Mathematical
// Functions, formula 7.1.26: erfc(x) = (a1 t + a2 t^2 + ... + a5 t^5) e^(-x^2),
// t = 1 / (1 + p x), x >= 0, absolute error <= 1.5e-7.  With
// h = erfc(|z| / sqrt 2) / 2, Phi(z) = h for z < 0 and 1 - h otherwise (no
// cancellation in the negative tail).  One reciprocal, one exp2 and a dozen
// FMA-class operations, about half the library erff; in float32 the result is
// within 4.3e-7 of the exact GELU for |z| <= 12, as close as erff-based float32.
__device__ __forceinline__ float act_gelu(float z) {
  const float x = fabsf(z) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, x, 1.0f));
  float poly = fmaf(1.061405429f, t, -1.453152027f);
  poly = fmaf(poly, t, 1.421413741f);
  poly = fmaf(poly, t, -0.284496736f);
  poly = fmaf(poly, t, 0.254829592f);
  const float e = __builtin_amdgcn_exp2f(z * z * -0.72134752044448170f);  // e^(-z^2 / 2)
  const float h = 0.5f * poly * t * e;
  return z * (z >= 0.f ? 1.0f - h : h);
}

template <int ACT> __device__ __forceinline__ float apply_act(float z) {
  if constexpr (ACT == 0) return act_relu(z);
  else if constexpr (ACT == 1) return act_gelu(z);
  else return z;
}

// d/dz of GELU: Phi(z) + z phi(z), with the library erff and expf.
__device__ __forceinline__ float gelu_grad(float z) {
  const float cdf = 0.5f * (1.0f + erff(z * 0.70710678118654752f));
  const float pdf = expf(-0.5f * z * z) * 0.39894228040143268f;
  return fmaf(z, pdf, cdf);
}

// act'(z): ReLU's derivative (0 at the kink) or GELU's.
template <int ACT> __device__ __forceinline__ float act_grad(float z) {
  if constexpr (ACT == 0) return z > 0.f ? 1.f : 0.f;
  else return gelu_grad(z);
}

// Wave-wide reductions (wave64) built on cross-lane shuffles.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ int wave_inclusive_scan(int v, int lane) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    int w = __shfl_up(v, o, kWave);
    if (lane >= o) v += w;
  }
  return v;
}

// Renumber block b of nblk so that blocks b, b+8, b+16, ... (which the
// dispatcher places on one XCD, round robin) get consecutive ids.
__device__ __forceinline__ int xcd_major_id(int b, int nblk) {
  const int q = nblk / 8, r = nblk % 8;
  const int x = b % 8, j = b / 8;
  const int base = x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q;
  return base + j;
}

// ---- LDS stage rings fed by direct global->LDS loads ----
// Rows of 128 bytes (64 bf16); the 16-byte chunk index is XORed with
// (row / 2) % 8 so that sixteen consecutive rows read at one chunk position
// fall in distinct banks.
__device__ __forceinline__ int lds_swz(int row) { return (row >> 1) & 7; }

// Same for rows of CPR 16-byte chunks: 8 chunks (128-byte rows) XOR (row/2)%8,
// 4 chunks (64-byte rows) XOR (row/4)%4; either way sixteen consecutive rows
// at one chunk position cover sixteen distinct 16-byte bank groups.
template <int CPR>
__device__ __forceinline__ int lds_swz_n(int row) {
  if constexpr (CPR == 8) return (row >> 1) & 7;
  else return (row >> 2) & 3;
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// s_waitcnt vmcnt(n) for a wave-uniform n known only at run time (0 <= n < 64).
__device__ __forceinline__ void wait_vmcnt_dyn(int n) {
  switch (n) {
#define MOE_W1(i) case i: wait_vmcnt<i>(); break;
#define MOE_W4(i) MOE_W1(i) MOE_W1(i + 1) MOE_W1(i + 2) MOE_W1(i + 3)
#define MOE_W16(i) MOE_W4(i) MOE_W4(i + 4) MOE_W4(i + 8) MOE_W4(i + 12)
    MOE_W16(0) MOE_W16(16) MOE_W16(32) MOE_W16(48)
#undef MOE_W16
#undef MOE_W4
#undef MOE_W1
    default: wait_vmcnt<0>();
  }
}

typedef __attribute__((address_space(3))) void lds_void;

// Work-group barrier for the stage ring.  It must not drain the prefetched
// direct-to-LDS loads (a fenced __syncthreads() waits for all of them), so it
// is a bare s_barrier after this wave's own LDS reads have completed; the
// stage data itself is covered by the explicit memory-counter wait before it.
// LDS reads of a stage feed MFMAs of the same iteration, and the next LDS
// write to that slot is a load issued after the barrier, which the compiler
// does not move above it.
__device__ __forceinline__ void ring_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), other counters unconstrained
  __builtin_amdgcn_s_barrier();
}

}  // namespace moe
