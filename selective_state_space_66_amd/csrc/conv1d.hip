// conv1d.hip -- the Mamba block's short causal depthwise convolution (+ SiLU)
// for gfx950, over whole sequences and as one decoding step.
//
// "Mamba and selective state spaces" (zerotofrontier.app/ssm/mamba), "The
// Mamba block": x_t = SiLU(sum_{i<k} w_i * xt_{t-i} + b_conv), each channel
// with its own k taps, inputs before the sequence taken as zero.  Decoding
// keeps the last k - 1 inputs of the convolution per sequence, oldest first,
// and shifts them every step ("Decoding with a constant-size cache"; the
// window holds inputs, not outputs: "Where Mamba implementations go wrong").
//
// Both kernels move each input once and each output once; they are bound by
// HBM.  A thread owns VEC consecutive channels (one 8-byte bf16 or 16-byte
// fp32 access per token when VEC = 4) and, in the sequence kernel, a run of T
// tokens: it keeps the last K - 1 inputs of its channels in registers as a
// sliding window and reads the K - 1 inputs before its run once more (the
// halo, K - 1 of T + K - 1 loads).  A wave covers 64 * VEC consecutive
// channels of one token row, so every access is a contiguous 512- or
// 1024-byte segment.
#include "ssm_device.h"
#include "ssm_launch.h"

namespace ssm66 {

namespace {

constexpr int kConvT = 16;       // tokens per thread (sequence kernel)
constexpr int kConvWaves = 4;    // waves per block, along the tokens

template <typename IO, int VEC>
struct VecIO;
template <>
struct VecIO<float, 1> {
  static __device__ __forceinline__ void load(const float* p, float (&v)[1]) { v[0] = *p; }
  static __device__ __forceinline__ void store(float* p, const float (&v)[1]) { *p = v[0]; }
};
template <>
struct VecIO<float, 4> {
  static __device__ __forceinline__ void load(const float* p, float (&v)[4]) {
    const float4 q = *(const float4*)p;
    v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
  }
  static __device__ __forceinline__ void store(float* p, const float (&v)[4]) {
    *(float4*)p = make_float4(v[0], v[1], v[2], v[3]);
  }
};
template <>
struct VecIO<bf16_bits, 1> {
  static __device__ __forceinline__ void load(const bf16_bits* p, float (&v)[1]) {
    v[0] = to_f32(*p);
  }
  static __device__ __forceinline__ void store(bf16_bits* p, const float (&v)[1]) {
    store_io(p, v[0]);
  }
};
template <>
struct VecIO<bf16_bits, 4> {
  static __device__ __forceinline__ void load(const bf16_bits* p, float (&v)[4]) {
    const uint2 q = *(const uint2*)p;
    v[0] = __uint_as_float(q.x << 16);
    v[1] = __uint_as_float(q.x & 0xffff0000u);
    v[2] = __uint_as_float(q.y << 16);
    v[3] = __uint_as_float(q.y & 0xffff0000u);
  }
  static __device__ __forceinline__ void store(bf16_bits* p, const float (&v)[4]) {
    uint2 q;
    q.x = pack_bf16x2(v[0], v[1]);
    q.y = pack_bf16x2(v[2], v[3]);
    *(uint2*)p = q;
  }
};

__device__ __forceinline__ float conv_act(float v, bool silu) { return silu ? silu_f(v) : v; }

// One thread: channels [c0, c0 + VEC) of batch entry b, tokens [t0, t0 + T).
// win[j] holds the input j + 1 steps back (j = 0 newest).
template <typename IO, int K, int VEC>
__global__ __launch_bounds__(64 * kConvWaves) void conv1d_fwd_kernel(
    const IO* __restrict__ x, const float* __restrict__ w, const float* __restrict__ bias,
    const IO* __restrict__ state_in, const int32_t* __restrict__ seq_lens,
    const uint8_t* __restrict__ reset, IO* __restrict__ out, IO* __restrict__ state_out,
    const int64_t L, const int64_t dim, const int64_t nvec, const int silu) {
  using V = VecIO<IO, VEC>;
  const int64_t cv = (int64_t)blockIdx.x * 64 + (threadIdx.x & 63);
  const int64_t t0 = ((int64_t)blockIdx.y * kConvWaves + (threadIdx.x >> 6)) * kConvT;
  const int64_t b = blockIdx.z;
  if (cv >= nvec || t0 >= (L > 0 ? L : 1)) return;
  const int64_t c0 = cv * VEC;
  int64_t len = L;
  if (seq_lens) {
    const int64_t sl = seq_lens[b];
    len = sl < 0 ? 0 : (sl < L ? sl : L);
  }

  float wt[VEC][K], bs[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) {
#pragma unroll
    for (int i = 0; i < K; ++i) wt[v][i] = w[(c0 + v) * K + i];
    bs[v] = bias ? bias[c0 + v] : 0.0f;
  }

  // ---- the window before t0: replay inputs t0 - (K - 1) .. t0 - 1 (negative
  // positions come from state_in), clearing at document starts
  float win[K > 1 ? K - 1 : 1][VEC];
#pragma unroll
  for (int j = 0; j < K - 1; ++j)
#pragma unroll
    for (int v = 0; v < VEC; ++v) win[j][v] = 0.0f;
#pragma unroll
  for (int q = K - 1; q >= 1; --q) {
    const int64_t s = t0 - q;
    // positions at or past len occur only when len < t0 (all outputs zero)
    const bool use = s < 0 || s < len;
    float in[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) in[v] = 0.0f;
    if (s >= 0 && use) {
      if (reset && reset[b * L + s]) {
#pragma unroll
        for (int j = 0; j < K - 1; ++j)
#pragma unroll
          for (int v = 0; v < VEC; ++v) win[j][v] = 0.0f;
      }
      V::load(x + (b * L + s) * dim + c0, in);
    } else if (s < 0 && state_in) {
      V::load(state_in + (b * (K - 1) + (K - 1 + s)) * dim + c0, in);
    }
    if (use) {
#pragma unroll
      for (int j = K - 2; j >= 1; --j)
#pragma unroll
        for (int v = 0; v < VEC; ++v) win[j][v] = win[j - 1][v];
#pragma unroll
      for (int v = 0; v < VEC; ++v) win[0][v] = in[v];
    }
  }

  auto write_state = [&]() {
    if (!state_out) return;
#pragma unroll
    for (int j = 0; j < K - 1; ++j) {
      float o[VEC];
#pragma unroll
      for (int v = 0; v < VEC; ++v) o[v] = win[K - 2 - j][v];  // oldest first
      V::store(state_out + (b * (K - 1) + j) * dim + c0, o);
    }
  };
  if (len == 0 && t0 == 0) write_state();

  // ---- this thread's tokens: all loads first, then the sliding window
  const int nt = (int)(L - t0 < kConvT ? L - t0 : kConvT);
  float xin[kConvT][VEC];
#pragma unroll
  for (int i = 0; i < kConvT; ++i) {
    if (i < nt && t0 + i < len) V::load(x + (b * L + t0 + i) * dim + c0, xin[i]);
  }
  const bool has_reset = reset != nullptr;
#pragma unroll
  for (int i = 0; i < kConvT; ++i) {
    if (i < nt) {
    const int64_t t = t0 + i;
    float o[VEC];
    if (t >= len) {
#pragma unroll
      for (int v = 0; v < VEC; ++v) o[v] = 0.0f;  // padding outputs 0
    } else {
      if (has_reset && reset[b * L + t]) {
#pragma unroll
        for (int j = 0; j < K - 1; ++j)
#pragma unroll
          for (int v = 0; v < VEC; ++v) win[j][v] = 0.0f;
      }
#pragma unroll
      for (int v = 0; v < VEC; ++v) {
        float acc = fmaf(wt[v][0], xin[i][v], bs[v]);
#pragma unroll
        for (int j = 1; j < K; ++j) acc = fmaf(wt[v][j], win[j - 1][v], acc);
        o[v] = conv_act(acc, silu);
      }
#pragma unroll
      for (int j = K - 2; j >= 1; --j)
#pragma unroll
        for (int v = 0; v < VEC; ++v) win[j][v] = win[j - 1][v];
      if constexpr (K > 1) {
#pragma unroll
        for (int v = 0; v < VEC; ++v) win[0][v] = xin[i][v];
      }
      if (t == len - 1) write_state();
    }
    V::store(out + (b * L + t) * dim + c0, o);
    }
  }
}

// One decoding step: out = act(w_0 x + sum_{i>=1} w_i window[K-1-i] + b), then
// the window drops its oldest input and appends x.
template <typename IO, int K, int VEC>
__global__ __launch_bounds__(256) void conv1d_step_kernel(
    IO* __restrict__ window, const IO* __restrict__ x, const float* __restrict__ w,
    const float* __restrict__ bias, IO* __restrict__ out, const int64_t batch, const int64_t dim,
    const int64_t nvec, const int silu) {
  using V = VecIO<IO, VEC>;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= batch * nvec) return;
  const int64_t b = gid / nvec;
  const int64_t c0 = (gid - b * nvec) * VEC;
  float xt[VEC], win[K > 1 ? K - 1 : 1][VEC];  // win[j]: j = 0 oldest
  V::load(x + b * dim + c0, xt);
#pragma unroll
  for (int j = 0; j < K - 1; ++j) V::load(window + (b * (K - 1) + j) * dim + c0, win[j]);
  float o[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) {
    float acc = fmaf(w[(c0 + v) * K], xt[v], bias ? bias[c0 + v] : 0.0f);
#pragma unroll
    for (int i = 1; i < K; ++i) acc = fmaf(w[(c0 + v) * K + i], win[K - 1 - i][v], acc);
    o[v] = conv_act(acc, silu);
  }
  V::store(out + b * dim + c0, o);
  // shift: the window drops its oldest input and appends x
#pragma unroll
  for (int j = 0; j + 1 < K - 1; ++j) V::store(window + (b * (K - 1) + j) * dim + c0, win[j + 1]);
  if constexpr (K > 1) V::store(window + (b * (K - 1) + (K - 2)) * dim + c0, xt);
}

template <typename IO, int K, int VEC>
hipError_t fwd_launch(const ConvParams& p, hipStream_t stream) {
  const int64_t nvec = p.dim / VEC;
  const int64_t tchunks = (p.L + (int64_t)kConvT * kConvWaves - 1) / ((int64_t)kConvT * kConvWaves);
  const dim3 grid((unsigned)((nvec + 63) / 64), (unsigned)(tchunks > 0 ? tchunks : 1),
                  (unsigned)p.batch);
  hipLaunchKernelGGL((conv1d_fwd_kernel<IO, K, VEC>), grid, dim3(64 * kConvWaves), 0, stream,
                     (const IO*)p.x, p.w, p.bias, (const IO*)p.state_in, p.seq_lens, p.reset,
                     (IO*)p.out, (IO*)p.state_out, p.L, p.dim, nvec, p.silu);
  return hipGetLastError();
}

template <typename IO, int K, int VEC>
hipError_t step_launch(const ConvParams& p, hipStream_t stream) {
  const int64_t nvec = p.dim / VEC;
  const int64_t n = p.batch * nvec;
  hipLaunchKernelGGL((conv1d_step_kernel<IO, K, VEC>), dim3((unsigned)((n + 255) / 256)),
                     dim3(256), 0, stream, (IO*)p.state_out, (const IO*)p.x, p.w, p.bias,
                     (IO*)p.out, p.batch, p.dim, nvec, p.silu);
  return hipGetLastError();
}

template <typename IO, int VEC>
hipError_t by_width(const ConvParams& p, bool step, hipStream_t stream) {
  switch (p.k) {
    case 1: return step ? step_launch<IO, 1, VEC>(p, stream) : fwd_launch<IO, 1, VEC>(p, stream);
    case 2: return step ? step_launch<IO, 2, VEC>(p, stream) : fwd_launch<IO, 2, VEC>(p, stream);
    case 3: return step ? step_launch<IO, 3, VEC>(p, stream) : fwd_launch<IO, 3, VEC>(p, stream);
    case 4: return step ? step_launch<IO, 4, VEC>(p, stream) : fwd_launch<IO, 4, VEC>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename IO>
hipError_t by_vec(const ConvParams& p, bool vec4, bool step, hipStream_t stream) {
  return vec4 ? by_width<IO, 4>(p, step, stream) : by_width<IO, 1>(p, step, stream);
}

}  // namespace

hipError_t launch_conv1d(const ConvParams& p, int io_dtype, bool vec4, bool step,
                         hipStream_t stream) {
  if (io_dtype == 1) return by_vec<bf16_bits>(p, vec4, step, stream);
  return by_vec<float>(p, vec4, step, stream);
}

}  // namespace ssm66
