// ssm_launch.h -- internal interface between the C-ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm66 {

struct ScanParams {
  const void* u;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;           // nullable
  const void* z;            // nullable
  const float* delta_bias;  // nullable
  const float* h0;          // nullable: initial state (batch, dim, N)
  const int32_t* seq_lens;  // nullable: real tokens per sequence (batch)
  const uint8_t* reset;     // nullable: document starts (batch, L)
  void* y;
  float* last_state;  // nullable; may be the same buffer as h0
  int64_t batch, L, dim, N;
  int softplus;
};

struct StepParams {
  float* state;
  const void* u;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;
  const void* z;
  const float* delta_bias;
  void* y;
  int64_t batch, dim, N;
  int softplus;
};

// G = states per thread, NG = state groups per channel, G * NG >= N.
// Supported (G, NG): (4, 4), (2, 8), (1, 16) for up to 16 states, (2, 4) and (1, 4).
hipError_t launch_scan_fwd(const ScanParams& p, int io_dtype, int G, int NG, bool zoh, bool gate,
                           hipStream_t stream);
hipError_t launch_step(const StepParams& p, int io_dtype, bool zoh, bool gate, hipStream_t stream);

}  // namespace ssm66
