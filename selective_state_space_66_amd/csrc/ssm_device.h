// ssm_device.h -- device helpers shared by the scan and step kernels (gfx950).
//
// Element access for the two I/O dtypes, the softplus step size and the SiLU
// gate, written on the hardware transcendental unit (v_exp_f32 is 2^x,
// v_log_f32 is log2 x, v_rcp_f32 is 1/x).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm66 {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;

// bf16 travels as its raw 16-bit pattern; the fp32 value is the pattern in the
// upper half of the word (exact).
using bf16_bits = uint16_t;

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16_bits v) { return __uint_as_float((uint32_t)v << 16); }

__device__ __forceinline__ void store_io(float* p, float v) { *p = v; }
// round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ void store_io(bf16_bits* p, float v) {
  *p = __builtin_bit_cast(uint16_t, (__bf16)v);
}

// two floats -> two bf16 (round to nearest even) in one word, a in the low half
// (a two-element vector conversion: one v_cvt_pk_bf16_f32 instead of two
// conversions, a shift and an or)
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __attribute__((ext_vector_type(2))) float f32x2_t;
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// Barrier for data exchanged through LDS only.  __syncthreads() also fences
// global memory at workgroup scope, which makes every wave wait for all of its
// outstanding global loads (vmcnt(0)) -- including loads issued ahead of time
// for the next chunk.  Here each wave waits for its own LDS operations
// (lgkmcnt(0); vmcnt and expcnt left alone), then meets the others; the signal
// fence stops the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float rcp_hw(float x) { return __builtin_amdgcn_rcpf(x); }

// softplus(v) = log(1 + e^v) = max(v, 0) + log(1 + e^-|v|): the exponential
// is at most 1, so nothing overflows and no threshold is needed.  w = 1 + e is
// rounded; r = (w - 1) - e is that rounding error, exactly (Sterbenz), and
// log(1 + e) = log(w) - r / w ~ log(w) - r keeps small step sizes accurate in
// relative terms, not only to 6e-8 absolute.
__device__ __forceinline__ float softplus_f(float v) {
  const float e = exp2_hw(-fabsf(v) * kLog2e);
  const float w = 1.0f + e;
  const float r = (w - 1.0f) - e;
  return fmaf(log2_hw(w), kLn2, fmaxf(v, 0.0f) - r);
}

// SiLU(z) = z * sigmoid(z) = z / (1 + e^-z); z -> -inf gives -0, not NaN.
__device__ __forceinline__ float silu_f(float z) {
  return z * rcp_hw(1.0f + exp2_hw(-z * kLog2e));
}

// phi(k) = (e^k - 1) / k, the zero-order-hold factor bbar = Delta B phi(Delta A).
// Series below |k| = 1/2 (error < 2e-7 relative), the quotient above it.
__device__ __forceinline__ float zoh_phi(float k, float ek) {
  const float s = fmaf(k, fmaf(k, fmaf(k, fmaf(k, fmaf(k, fmaf(k, 1.0f / 5040.0f, 1.0f / 720.0f),
                                                        1.0f / 120.0f), 1.0f / 24.0f), 1.0f / 6.0f),
                               0.5f), 1.0f);
  return fabsf(k) < 0.5f ? s : (ek - 1.0f) * rcp_hw(k);
}

}  // namespace ssm66
