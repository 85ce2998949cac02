// Shared device helpers of the gfx950 kernels: storage types, conversions,
// wavefront reductions and the MFMA operand vector types.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vla {

typedef uint16_t bf16_t;  // raw bfloat16 bits

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2_t;

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float -> bfloat16, round to nearest even (NaN stays NaN)
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<bf16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

// element access in the activation storage type
template <typename T> struct St;
template <> struct St<float> {
  static __device__ __forceinline__ float ld(const float* p, size_t i) { return p[i]; }
  static __device__ __forceinline__ void st(float* p, size_t i, float v) { p[i] = v; }
};
template <> struct St<bf16_t> {
  static __device__ __forceinline__ float ld(const bf16_t* p, size_t i) { return bf16_to_f32(p[i]); }
  static __device__ __forceinline__ void st(bf16_t* p, size_t i, float v) { p[i] = f32_to_bf16(v); }
};

// the value of the lane K places away inside its row of 16 (DPP row rotation)
template <int K>
__device__ __forceinline__ float row_ror(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x120 + K, 0xF, 0xF, false));
}
// sum / max over a whole wavefront (every lane active) with no LDS traffic: lanes
// l ^ 32 and l ^ 16 by the row-swap permutes, then rotations by 8, 4, 2 and 1 inside
// each row of 16 (after the xor-8 step the values repeat with period 8 in a row, so
// each rotation pairs the values the xor butterfly would: the same operations,
// every lane the same result)
__device__ __forceinline__ float wave_sum(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(b[0]) + __uint_as_float(b[1]);
  v += row_ror<8>(v);
  v += row_ror<4>(v);
  v += row_ror<2>(v);
  return v + row_ror<1>(v);
}
__device__ __forceinline__ float wave_max(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
  v = fmaxf(v, row_ror<8>(v));
  v = fmaxf(v, row_ror<4>(v));
  v = fmaxf(v, row_ror<2>(v));
  return fmaxf(v, row_ror<1>(v));
}
// the two 32-bit halves of a double, and back
__device__ __forceinline__ void split_d(double x, uint32_t& lo, uint32_t& hi) {
  const unsigned long long u = __builtin_bit_cast(unsigned long long, x);
  lo = (uint32_t)u;
  hi = (uint32_t)(u >> 32);
}
__device__ __forceinline__ double join_d(uint32_t lo, uint32_t hi) {
  return __builtin_bit_cast(double, ((unsigned long long)hi << 32) | lo);
}
// v + v of the lane K places away inside its row of 16 (DPP row rotation)
template <int K>
__device__ __forceinline__ double row_ror_add(double v) {
  uint32_t lo, hi;
  split_d(v, lo, hi);
  const uint32_t plo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)lo, 0x120 + K, 0xF, 0xF, false);
  const uint32_t phi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)hi, 0x120 + K, 0xF, 0xF, false);
  return v + join_d(plo, phi);
}
// fp64 sum over a whole wavefront (every lane active) with no LDS traffic: lanes l ^ 32 and l ^ 16 by the
// row-swap permutes, then rotations by 8, 4, 2 and 1 inside each row of 16 (after
// the xor-8 step the values repeat with period 8 in a row, so each rotation pairs
// the values the xor butterfly would: the same additions, every lane the same sum)
__device__ __forceinline__ double wave_sum_d(double v) {
  uint32_t lo, hi;
  split_d(v, lo, hi);
  {
    const auto a = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
    const auto b = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
    v = join_d(a[0], b[0]) + join_d(a[1], b[1]);
  }
  split_d(v, lo, hi);
  {
    const auto a = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
    const auto b = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
    v = join_d(a[0], b[0]) + join_d(a[1], b[1]);
  }
  v = row_ror_add<8>(v);
  v = row_ror_add<4>(v);
  v = row_ror_add<2>(v);
  return row_ror_add<1>(v);
}

// wait until at most steps * STEP of this wavefront's vector-memory operations are
// outstanding (vector loads, including direct-to-LDS ones, count in issue order)
template <int STEP>
__device__ __forceinline__ void wait_vmcnt_steps(int steps) {
  // s_waitcnt simm16: vmcnt[3:0], expcnt[6:4] (7 = no wait), lgkmcnt[11:8] (15 = no
  // wait), vmcnt[5:4] in [15:14]
#define VLA_WAITVM(v) __builtin_amdgcn_s_waitcnt(((v) & 0xF) | 0x70 | 0xF00 | (((v) >> 4) << 14))
  switch (steps) {
    case 0: VLA_WAITVM(0); break;
    case 1: VLA_WAITVM(STEP); break;
    case 2: VLA_WAITVM(2 * STEP); break;
    case 3: VLA_WAITVM(3 * STEP); break;
    case 4: VLA_WAITVM(4 * STEP); break;
    case 5: VLA_WAITVM(5 * STEP); break;
    case 6: VLA_WAITVM(6 * STEP); break;
    default: VLA_WAITVM(0); break;
  }
#undef VLA_WAITVM
}

// two floats -> packed bfloat16 pair (round to nearest even; one v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf2_t __attribute__((ext_vector_type(2)));
  typedef float f2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2_t){lo, hi}, bf2_t));
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }
// exact GELU: z * Phi(z) = z/2 * (1 + erf(z / sqrt 2))
__device__ __forceinline__ float gelu_erf(float z) { return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f)); }
// gated FFN activation of a (gate, up) pair: SwiGLU (glu 0) or GeGLU (glu 1)
__device__ __forceinline__ float glu_act(int glu, float gate, float up) {
  return (glu ? gelu_erf(gate) : silu(gate)) * up;
}

// gated activation with the hardware exp2 and reciprocal (no IEEE divide, no
// branches): SwiGLU silu(g) * u, or GeGLU gelu(g) * u with the exact-erf GELU
// INT4 offset-binary unpacking: the two nibbles of t at bits 0..3 and 16..19
// (two's-complement codes q) as a bf16 pair of 128 + (q + 8), in one v_bitop3:
// (t & 0x000F000F) ^ 0x43084308 keeps the nibbles, flips their sign bits and
// sets the exponent of 128 (truth table 0x6C = (a & c) ^ b)
__device__ __forceinline__ uint32_t w4_pair_bits(uint32_t t) {
  return __builtin_amdgcn_bitop3_b32(t, 0x43084308u, 0x000F000Fu, 0x6C);
}

template <bool GELU>
__device__ __forceinline__ float glu_fast(float g, float u) {
  if constexpr (GELU) return gelu_erf(g) * u;
  return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(g * -1.4426950408889634f)) * u;
}

// float -> bfloat16 bits, round to nearest even, in one v_cvt_pk_bf16_f32
__device__ __forceinline__ bf16_t bf16_rne(float v) {
  return static_cast<bf16_t>(pack_bf16x2(v, 0.0f) & 0xffffu);
}

// 8 bf16 values held in a 16-byte register quad, unpacked to fp32
__device__ __forceinline__ void unpack8(const u32x4_t& w, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

}  // namespace vla
