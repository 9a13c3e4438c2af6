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
  float* ckpt;        // nullable: the state before every 16th token (batch, ceil(L/16), dim, N)
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

struct ScanBwdParams {
  const void *u, *delta, *B, *C, *z, *dy;     // io dtype; z nullable
  const float *A, *D, *delta_bias, *h0, *dlast;  // D, delta_bias, h0, dlast nullable
  const int32_t* seq_lens;                     // nullable: real tokens per sequence
  const uint8_t* reset;                        // nullable: document starts (batch, L)
  void *du, *ddelta, *dB, *dC, *dz;           // io dtype; dz nullable
  float *dA, *dD, *ddelta_bias, *dh0;          // dD, ddelta_bias, dh0 nullable
  void* workspace;                             // scan_bwd_workspace_bytes(...) bytes
  const float* ckpt;                           // nullable: checkpoints written by the forward
  int64_t batch, L, dim, N;
  int softplus;
};

struct SSDParams {
  const void *x, *B, *C, *z;  // bf16; z nullable
  const float *dt, *A, *D, *dt_bias, *h0;  // D, dt_bias, h0 nullable
  void* y;
  float* last_state;  // nullable
  int64_t batch, L, nheads, P, N;
  int softplus;
};

struct ConvParams {
  const void* x;            // (batch, L, dim) io dtype; (batch, dim) for a step
  const float* w;           // (dim, k): w[c * k + i] multiplies the input i steps back
  const float* bias;        // nullable (dim)
  const void* state_in;     // nullable window before the sequence (batch, k - 1, dim)
  const int32_t* seq_lens;  // nullable (batch)
  const uint8_t* reset;     // nullable (batch, L)
  void* out;
  void* state_out;          // nullable window after the last real token; a step's window (in/out)
  int64_t batch, L, dim, k;
  int silu;
};

// G = states per thread, NG = state groups per channel, G * NG >= N.
// Supported (G, NG): (4, 4), (2, 8), (1, 16) for up to 16 states, (2, 4) and (1, 4).
hipError_t launch_scan_fwd(const ScanParams& p, int io_dtype, int G, int NG, bool zoh, bool gate,
                           hipStream_t stream);
// step = false: the sequence kernel; true: one decoding step.  vec4: dim is a
// multiple of 4 and the io pointers are aligned to 4 elements.
// The convolution's backward pass: gradients of x, w, bias and the
// carried-in window given dout and the gradient of the window handed on.
struct ConvBwdParams {
  const void* x;            // (batch, L, dim) io dtype
  const float* w;           // (dim, k)
  const float* bias;        // nullable (dim)
  const void* state_in;     // nullable (batch, k - 1, dim)
  const int32_t* seq_lens;  // nullable (batch)
  const uint8_t* reset;     // nullable (batch, L)
  const void* dout;         // (batch, L, dim) io dtype
  const void* dstate_out;   // nullable (batch, k - 1, dim) io dtype
  void* dx;                 // (batch, L, dim) io dtype
  float* dw;                // (dim, k)
  float* dbias;             // nullable (dim)
  void* dstate_in;          // nullable (batch, k - 1, dim) io dtype; written when state_in is given
  void* workspace;          // conv1d_bwd_workspace_bytes(...) bytes
  int64_t batch, L, dim, k;
  int silu;
};
int64_t conv1d_bwd_spans(int64_t L);
size_t conv1d_bwd_workspace_bytes(int64_t batch, int64_t L, int64_t dim, int64_t k);
hipError_t launch_conv1d_bwd(const ConvBwdParams& q, int io_dtype, bool vec4, hipStream_t stream);

hipError_t launch_conv1d(const ConvParams& p, int io_dtype, bool vec4, bool step,
                         hipStream_t stream);
size_t scan_bwd_ckpt_bytes(int64_t batch, int64_t L, int64_t dim, int64_t N);
size_t scan_bwd_workspace_bytes(int64_t batch, int64_t L, int64_t dim, int64_t N);
hipError_t launch_scan_bwd(const ScanBwdParams& p, int io_dtype, bool zoh, bool gate,
                           hipStream_t stream);
// P a multiple of 16, N in {64, 128}, bf16 io; 16-byte aligned x, z, y, B, C.
// The time-parallel scan (lanes hold tokens; associative pair scan).
hipError_t launch_scan_tpar(const ScanParams& p, int io_dtype, bool zoh, bool gate,
                            hipStream_t stream);
// The time-parallel scan with one wave (channels_per_wave 1) or a row of 16
// lanes (channels_per_wave 4) per (batch, channel) row and four consecutive
// tokens per lane (wide layers).
hipError_t launch_scan_wave(const ScanParams& p, int io_dtype, bool zoh, bool gate,
                            int channels_per_wave, hipStream_t stream);
hipError_t launch_ssd_fwd(const SSDParams& p, bool zoh, bool gate, hipStream_t stream);
hipError_t launch_step(const StepParams& p, int io_dtype, bool zoh, bool gate, hipStream_t stream);

// Issue-rate probes (probe.hip): blocks x 256 lanes, iters iterations of 8
// FMAs, 8 exponentials, or 8 x (exponential + 4 FMAs); sink holds one float
// per lane.
constexpr int kAluProbeFma = 0;
constexpr int kAluProbeExp = 1;
constexpr int kAluProbeMix = 2;
hipError_t launch_alu_probe(int op, float* sink, int64_t blocks, int iters, hipStream_t stream);

}  // namespace ssm66
