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
// HBM.  A thread owns VEC = 4 consecutive channels (one 8-byte bf16 or 16-byte
// fp32 access per token) and, in the sequence kernel, a run of T
// tokens: it keeps the last K - 1 inputs of its channels in registers as a
// sliding window and reads the K - 1 inputs before its run once more (the
// halo, mostly served by L2: the neighbouring run read those rows).  A wave
// covers 256 consecutive channels of one token row, so every access is a
// contiguous 512- or 1024-byte segment.  All loads of a thread are issued
// before the first is used.
#include "ssm_device.h"
#include "ssm_launch.h"

namespace ssm66 {

namespace {

constexpr int kConvT = 8;        // tokens per thread (sequence kernel)
constexpr int kConvWaves = 4;    // waves per block, along the tokens

// VEC consecutive io elements: Raw is what one access moves (kept raw in
// registers until used: a bf16 word holds two values), unpack turns it into
// fp32, store rounds fp32 back (bf16: nearest even).
template <typename IO, int VEC>
struct VecIO;
template <>
struct VecIO<float, 1> {
  using Raw = float;
  static __device__ __forceinline__ Raw load_raw(const float* p) { return *p; }
  static __device__ __forceinline__ void unpack(Raw r, float (&v)[1]) { v[0] = r; }
  static __device__ __forceinline__ void store(float* p, const float (&v)[1]) { *p = v[0]; }
};
template <>
struct VecIO<float, 4> {
  using Raw = float4;
  static __device__ __forceinline__ Raw load_raw(const float* p) { return *(const float4*)p; }
  static __device__ __forceinline__ void unpack(Raw q, float (&v)[4]) {
    v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
  }
  static __device__ __forceinline__ void store(float* p, const float (&v)[4]) {
    *(float4*)p = make_float4(v[0], v[1], v[2], v[3]);
  }
};
template <>
struct VecIO<bf16_bits, 1> {
  using Raw = uint32_t;
  static __device__ __forceinline__ Raw load_raw(const bf16_bits* p) { return *p; }
  static __device__ __forceinline__ void unpack(Raw r, float (&v)[1]) {
    v[0] = __uint_as_float(r << 16);
  }
  static __device__ __forceinline__ void store(bf16_bits* p, const float (&v)[1]) {
    store_io(p, v[0]);
  }
};
template <>
struct VecIO<bf16_bits, 4> {
  using Raw = uint2;
  static __device__ __forceinline__ Raw load_raw(const bf16_bits* p) { return *(const uint2*)p; }
  static __device__ __forceinline__ void unpack(Raw q, float (&v)[4]) {
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
template <typename IO, int VEC>
__device__ __forceinline__ void vload(const IO* p, float (&v)[VEC]) {
  VecIO<IO, VEC>::unpack(VecIO<IO, VEC>::load_raw(p), v);
}

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

  // optional inputs are read through a valid stand-in pointer and masked, so
  // that no load sits behind a branch (a branch around a load makes the
  // compiler wait for it on the spot)
  const float* bias_src = bias ? bias : w;
  float wt[VEC][K], bs[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) {
#pragma unroll
    for (int i = 0; i < K; ++i) wt[v][i] = w[(c0 + v) * K + i];
    const float bv = bias_src[c0 + v];
    bs[v] = bias ? bv : 0.0f;
  }

  // ---- every load first, unconditionally, through addresses clamped into the
  // tensors (values of padded or out-of-range positions are then masked), so
  // that all of them are in flight together
  if (L == 0) {  // no tokens: the window carries over (thread t0 == 0 only)
    float win[K > 1 ? K - 1 : 1][VEC];
#pragma unroll
    for (int j = 0; j < K - 1; ++j) {
#pragma unroll
      for (int v = 0; v < VEC; ++v) win[j][v] = 0.0f;
      if (state_in) vload<IO, VEC>(state_in + (b * (K - 1) + j) * dim + c0, win[j]);
      if (state_out) V::store(state_out + (b * (K - 1) + j) * dim + c0, win[j]);
    }
    return;
  }
  auto row = [&](int64_t t) -> int64_t { return t < 0 ? 0 : (t < L ? t : L - 1); };
  // reset flags: x holds at least batch * L bytes, so it stands in when reset is NULL
  const uint8_t* rsrc = reset ? reset : (const uint8_t*)x;
  const int rmask = reset ? 0xff : 0;
  typename V::Raw xh[K > 1 ? K - 1 : 1];  // xh[q - 1]: the input at t0 - q
  int rh[K > 1 ? K - 1 : 1];
#pragma unroll
  for (int q = 1; q < K; ++q) {
    const int64_t s = t0 - q;
    const IO* src = x + (b * L + row(s)) * dim + c0;
    if (s < 0 && state_in) src = state_in + (b * (K - 1) + (K - 1 + s)) * dim + c0;
    xh[q - 1] = V::load_raw(src);
    rh[q - 1] = (int)rsrc[b * L + row(s)] & rmask;
  }
  typename V::Raw xr[kConvT];
  int rf[kConvT];
#pragma unroll
  for (int i = 0; i < kConvT; ++i) {
    xr[i] = V::load_raw(x + (b * L + row(t0 + i)) * dim + c0);
    rf[i] = (int)rsrc[b * L + row(t0 + i)] & rmask;
  }

  // ---- the window before t0: replay inputs t0 - (K - 1) .. t0 - 1 (negative
  // positions from state_in, or zero), clearing at document starts
  float win[K > 1 ? K - 1 : 1][VEC];
#pragma unroll
  for (int j = 0; j < K - 1; ++j)
#pragma unroll
    for (int v = 0; v < VEC; ++v) win[j][v] = 0.0f;
#pragma unroll
  for (int q = K - 1; q >= 1; --q) {
    const int64_t s = t0 - q;
    // positions at or past len occur only when len < t0 (all outputs zero)
    if (s < 0 || s < len) {
      const bool clear = s >= 0 && rh[q - 1] != 0;
      const bool zero = s < 0 && !state_in;
      float xv[VEC];
      V::unpack(xh[q - 1], xv);
#pragma unroll
      for (int j = K - 2; j >= 1; --j)
#pragma unroll
        for (int v = 0; v < VEC; ++v) win[j][v] = clear ? 0.0f : win[j - 1][v];
#pragma unroll
      for (int v = 0; v < VEC; ++v) win[0][v] = zero ? 0.0f : xv[v];
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

  // ---- this thread's tokens, through the sliding window
  const int nt = (int)(L - t0 < kConvT ? L - t0 : kConvT);
#pragma unroll
  for (int i = 0; i < kConvT; ++i) {
    if (i < nt) {
      const int64_t t = t0 + i;
      const bool live = t < len;
      const bool clear = live && rf[i] != 0;  // a document starts at t
      float xin[VEC];
      V::unpack(xr[i], xin);
      float o[VEC];
#pragma unroll
      for (int v = 0; v < VEC; ++v) {
        float acc = fmaf(wt[v][0], xin[v], bs[v]);
#pragma unroll
        for (int j = 1; j < K; ++j) acc = fmaf(wt[v][j], clear ? 0.0f : win[j - 1][v], acc);
        o[v] = live ? conv_act(acc, silu) : 0.0f;  // padding outputs 0
      }
      if (live) {
#pragma unroll
        for (int j = K - 2; j >= 1; --j)
#pragma unroll
          for (int v = 0; v < VEC; ++v) win[j][v] = clear ? 0.0f : win[j - 1][v];
        if constexpr (K > 1) {
#pragma unroll
          for (int v = 0; v < VEC; ++v) win[0][v] = xin[v];
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
  vload<IO, VEC>(x + b * dim + c0, xt);
#pragma unroll
  for (int j = 0; j < K - 1; ++j) vload<IO, VEC>(window + (b * (K - 1) + j) * dim + c0, win[j]);
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

// Four channels per thread where the channels and pointers allow (8-byte bf16
// or 16-byte fp32 accesses); else one.  Measured on the Mamba-130M layer's
// convolution: 8 tokens x 4 channels per thread, 4 waves per block, beats 16
// or 32 tokens (fewer waves in flight) and 16-byte bf16 accesses (more
// registers, half the occupancy).
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
