// probe.hip -- issue-rate probes for the scan's ALU roofline (gfx950).
//
// The scan is bound by plain VALU issue and by the transcendental unit, not
// by HBM ("Mamba and selective state spaces", "Why the scan must be fused":
// at N = 16 the exponentials, one per state update, set the floor).  Its
// roofline therefore needs two rates the published specification does not
// give per instruction: how many fp32 FMA lane-operations and how many
// v_exp_f32 lane-operations the chip completes per second, and what one
// exponential costs inside a stream of FMAs.  These kernels measure them.
//
// Each lane runs 8 independent dependency chains (enough, with 8 waves per
// SIMD, to hide every latency) of one of three bodies per iteration:
//   kFma : 8 x v_fma_f32                   x = x * a + b
//   kExp : 8 x v_exp_f32                   x = 2^(-x)  (negation is a free
//                                          source modifier; the chain
//                                          converges to a fixed point, so no
//                                          value overflows or goes denormal)
//   kMix : 8 x (v_exp_f32 then 4 x v_fma_f32), the exponential feeding the
//          FMAs of its own chain, as in a scan's state update
// and writes the sum of its chains to sink so that nothing is optimised away.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ssm_launch.h"

namespace ssm66 {

namespace {

constexpr int kChains = 8;

template <int OP>
__global__ __launch_bounds__(256) void alu_probe_kernel(float* __restrict__ sink, int iters,
                                                       float a, float b) {
  float x[kChains];
#pragma unroll
  for (int i = 0; i < kChains; ++i) x[i] = (float)(threadIdx.x & 63) * 1e-3f + 0.1f * (float)i;
#pragma unroll 4
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < kChains; ++i) {
      if constexpr (OP == kAluProbeFma) {
        x[i] = fmaf(x[i], a, b);
      } else if constexpr (OP == kAluProbeExp) {
        x[i] = __builtin_amdgcn_exp2f(-x[i]);
      } else {
        float e = __builtin_amdgcn_exp2f(-x[i]);
        e = fmaf(e, a, b);
        e = fmaf(e, a, b);
        e = fmaf(e, a, b);
        x[i] = fmaf(e, a, b);
      }
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < kChains; ++i) s += x[i];
  sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

hipError_t launch_alu_probe(int op, float* sink, int64_t blocks, int iters, hipStream_t stream) {
  // a and b keep the FMA chains bounded: |x| stays near b / (1 - a)
  const float a = 0.5f, b = 0.25f;
  const dim3 grid((unsigned)blocks), block(256);
  if (op == kAluProbeFma)
    hipLaunchKernelGGL(alu_probe_kernel<kAluProbeFma>, grid, block, 0, stream, sink, iters, a, b);
  else if (op == kAluProbeExp)
    hipLaunchKernelGGL(alu_probe_kernel<kAluProbeExp>, grid, block, 0, stream, sink, iters, a, b);
  else if (op == kAluProbeMix)
    hipLaunchKernelGGL(alu_probe_kernel<kAluProbeMix>, grid, block, 0, stream, sink, iters, a, b);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace ssm66
