// ssm_bwd.h -- arguments shared by the two backward kernels of the selective
// scan (scan_bwd.hip: states across threads, sequential in time;
// scan_bwd_wave.hip: time-parallel rows of 16 lanes) and the workspace layout
// they both write.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm66 {

struct BwdArgs {
  const void *u, *delta, *B, *C, *z, *dy;
  const float *A, *D, *bias, *h0, *dlast;
  const int32_t* seq_lens;  // nullable: real tokens per sequence
  const uint8_t* reset;     // nullable: document starts (batch, L)
  void *du, *ddelta, *dz;
  float* dh0;
  float* ckpt;    // (batch, nchunks, dim, N): the state at every 16th token
  int have_ckpt;  // ckpt was written by the forward: no forward sweep
  int split_fast; // another instance takes the fast blocks: each block runs in one
  float* pbc;     // (ntiles, 2, batch, L, N): dB, dC summed over a tile's 16 channels
  float* pA;      // (batch, dim, N)
  float* pDb;     // (2, batch, dim)
  int64_t batch, L, dim, N, ntiles, nchunks;
  int softplus, want_dz;
};

// The time-parallel backward: ZOH, N = 16, no document starts, dim a multiple
// of 16 and the (token, channel) tensors 16-byte aligned.  Its blocks own the
// 16-channel tiles whose states all have |A| >= 1/2 and leave the others.
hipError_t launch_scan_bwd_wave(const BwdArgs& a, bool bf16_io, bool gate, hipStream_t stream);

}  // namespace ssm66
