// Shared device helpers for the gfx950 kernels: bf16 bit conversions, vector types, wave reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint16_t bf16_t;  // raw bf16 bits in memory
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

#define WAN_DEV __device__ __forceinline__

WAN_DEV float bf16_to_f32(bf16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// fp32 -> bf16, round to nearest, ties to even (hardware conversion).
WAN_DEV bf16_t f32_to_bf16(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// two fp32 -> packed bf16x2 (low half = a), round to nearest even: one v_cvt_pk_bf16_f32 on gfx950.
WAN_DEV uint32_t pack_bf16x2(float a, float b) {
  f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

WAN_DEV float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
WAN_DEV float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Workgroup barrier without the memory fence of __syncthreads (which makes the compiler wait for every
// outstanding global access, direct-to-LDS loads included): callers wait for what they need with
// s_waitcnt first.  The empty asm statements keep the compiler from moving memory accesses across.
WAN_DEV void block_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

WAN_DEV bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Wave-wide (64 lanes) reductions.
WAN_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
WAN_DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// GELU, tanh form.  0.5 u (1 + tanh z) equals u * sigmoid(2 z), z = sqrt(2/pi) (u + 0.044715 u^3).
// GELU, tanh form: 0.5 u (1 + tanh(z)), z = sqrt(2/pi) (u + 0.044715 u^3), evaluated as u * sigmoid(2z)
// = u / (1 + 2^(-2 z log2(e))) with the constants folded into one polynomial in u, v_exp_f32 and the
// hardware reciprocal (about 1 ulp of fp32; a full IEEE division costs ~10 instructions).  Saturates
// correctly: u -> -inf gives 2^(+inf) = inf and u * rcp(inf) = 0; u -> +inf gives u * rcp(1) = u.
WAN_DEV float gelu_tanh_f(float u) {
  constexpr float c1 = -2.0f * 0.7978845608028654f * 1.4426950408889634f;  // -2 sqrt(2/pi) log2(e)
  constexpr float c2 = c1 * 0.044715f;
  const float e = __builtin_amdgcn_exp2f(u * fmaf(c2, u * u, c1));
  return u * __builtin_amdgcn_rcpf(1.0f + e);
}

// SiLU: u * sigmoid(u) = u / (1 + 2^(-u log2(e))), same evaluation as above.
WAN_DEV float silu_f(float u) {
  return u * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(u * -1.4426950408889634f));
}

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }
