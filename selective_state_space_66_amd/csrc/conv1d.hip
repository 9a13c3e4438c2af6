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
  static __device__ __forceinline__ Raw bload(__amdgpu_buffer_rsrc_t r, uint32_t vo, uint32_t so) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)vo, (int)so, 0));
  }
  static __device__ __forceinline__ void unpack(Raw r, float (&v)[1]) { v[0] = r; }
  static __device__ __forceinline__ void store(float* p, const float (&v)[1]) { *p = v[0]; }
};
template <>
struct VecIO<float, 4> {
  using Raw = float4;
  static __device__ __forceinline__ Raw load_raw(const float* p) { return *(const float4*)p; }
  static __device__ __forceinline__ Raw bload(__amdgpu_buffer_rsrc_t r, uint32_t vo, uint32_t so) {
    typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;
    const u32x4_t q = __builtin_amdgcn_raw_buffer_load_b128(r, (int)vo, (int)so, 0);
    return make_float4(__uint_as_float(q[0]), __uint_as_float(q[1]), __uint_as_float(q[2]),
                       __uint_as_float(q[3]));
  }
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
  static __device__ __forceinline__ Raw bload(__amdgpu_buffer_rsrc_t r, uint32_t vo, uint32_t so) {
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)vo, (int)so, 0);
  }
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
  static __device__ __forceinline__ Raw bload(__amdgpu_buffer_rsrc_t r, uint32_t vo, uint32_t so) {
    typedef __attribute__((ext_vector_type(2))) unsigned int u32x2_t;
    const u32x2_t q = __builtin_amdgcn_raw_buffer_load_b64(r, (int)vo, (int)so, 0);
    return make_uint2(q[0], q[1]);
  }
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

// ---- backward pass.  The chain rule through the forward above, in gather
// form: with dpre_t = dout_t act'(pre_t) for the real tokens (0 past a length),
//   dx_s  = sum_i w_i dpre_{s+i} [s visible from s + i] (+ the gradient of the
//           window handed to decoding, where s is one of its inputs),
//   dw_i  = sum_t dpre_t xt_{t-i} [visible],   dbias = sum_t dpre_t,
// and the carried-in window's gradient from the first K - 1 tokens; "s
// visible from t" means no document starts in (s, t].  A thread owns VEC
// channels and kBwdRuns * kBwdT consecutive tokens, which it streams through
// one pass with sliding windows: it reads x from K - 1 tokens before them to
// K - 1 after, dout to K - 1 after, each row once, recomputes pre and dpre
// over them and the K - 1 after, and writes their dx.  dw and dbias are summed
// over a thread's tokens, then over the block's waves through LDS, into one
// partial row per block; a second kernel adds the rows in a fixed order.
constexpr int kBwdT = 8;       // positions per load block
// word 3 of a raw buffer resource (no stride, 32-bit data format)
constexpr int kConvBufferFlags = 0x00020000;
constexpr int kBwdRuns = 4;    // load blocks of tokens per thread
constexpr int kBwdSpan = kConvWaves * kBwdRuns * kBwdT;  // tokens per block (128)

struct ConvBwdArgs {
  const void *x, *state_in, *dout, *dstate_out;
  const float *w, *bias;
  const int32_t* seq_lens;
  const uint8_t* reset;
  void *dx, *dstate_in;
  float* partial;  // (batch * nspans, K + 1, dim)
  int64_t L, dim, nspans;
  int silu;
};

__device__ __forceinline__ float act_prime(float v, bool silu) {
  if (!silu) return 1.0f;
  const float sg = rcp_hw(1.0f + exp2_hw(-v * kLog2e));
  return sg * fmaf(v, 1.0f - sg, 1.0f);
}

template <typename IO, int K, int VEC>
__global__ __launch_bounds__(64 * kConvWaves) void conv1d_bwd_kernel(const ConvBwdArgs p) {
  using V = VecIO<IO, VEC>;
  __shared__ float red[kConvWaves][VEC * (K + 1)][64];

  const IO* __restrict__ x = (const IO*)p.x;
  const IO* __restrict__ dout = (const IO*)p.dout;
  const IO* __restrict__ sin = (const IO*)p.state_in;
  const IO* __restrict__ dso = (const IO*)p.dstate_out;
  const int64_t L = p.L, dim = p.dim, nvec = dim / VEC;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar run bounds
  const int64_t cv = (int64_t)blockIdx.x * 64 + lane;
  const bool cok = cv < nvec;
  const int64_t c0 = (cok ? cv : nvec - 1) * VEC;  // loads of idle lanes stay in bounds
  const int64_t span = blockIdx.y, b = blockIdx.z;
  int64_t len = L;
  if (p.seq_lens) {
    const int64_t sl = p.seq_lens[b];
    len = sl < 0 ? 0 : (sl < L ? sl : L);
  }
  // one buffer resource per tensor and sequence (the launch keeps a
  // sequence's bytes below 2^32): rows at scalar offsets, channels at the
  // lane's offset
  const uint32_t loff = (uint32_t)c0 * (uint32_t)sizeof(IO);
  const uint32_t rowb = (uint32_t)dim * (uint32_t)sizeof(IO);
  const __amdgpu_buffer_rsrc_t rx =
      __builtin_amdgcn_make_buffer_rsrc((void*)(x + b * L * dim), (short)0, -1, kConvBufferFlags);
  const __amdgpu_buffer_rsrc_t rd =
      __builtin_amdgcn_make_buffer_rsrc((void*)(dout + b * L * dim), (short)0, -1, kConvBufferFlags);
  const __amdgpu_buffer_rsrc_t rwin = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(sin ? sin + b * (K - 1) * dim : x), (short)0, -1, kConvBufferFlags);
  const bool silu = p.silu != 0;

  float wt[VEC][K], bs[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) {
#pragma unroll
    for (int i = 0; i < K; ++i) wt[v][i] = p.w[(c0 + v) * K + i];
    bs[v] = p.bias ? p.bias[c0 + v] : 0.0f;
  }
  float dw[VEC][K], db[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) {
    db[v] = 0.0f;
#pragma unroll
    for (int i = 0; i < K; ++i) dw[v][i] = 0.0f;
  }
  // the gradient of the window handed to decoding: entry j is the input at
  // len - (K - 1) + j
  auto dwo = [&](int64_t j, float (&o)[VEC]) {
    vload<IO, VEC>(dso + (b * (K - 1) + j) * dim + c0, o);
  };

  // ---- this thread's tokens: NT consecutive positions from s0 (the wave's
  // part of the block's span), streamed through one pass with sliding
  // windows.  At x-window index q (position s0 - (K - 1) + q):
  //   - x enters the window (xw[i] is x i positions back);
  //   - from q = K - 1 on, p = s0 + q - (K - 1): pre_p and dpre_p (zero past
  //     the length; dpw[i] is dpre i positions back), and the dw and dbias
  //     terms of p while p is one of this thread's tokens;
  //   - from q = 2 (K - 1) on, dx of s = p - (K - 1), one of its tokens.
  // The last K - 1 positions only complete dpre for the dx of the last
  // tokens.  Every row is loaded once, kBwdT positions ahead of its first use.
  constexpr int NT = kBwdRuns * kBwdT;             // tokens of a thread
  constexpr int NXT = NT + 2 * (K - 1);            // x positions
  constexpr int NDT = NT + (K - 1);                // dout positions
  static_assert(NXT <= 64, "document starts of a thread fit one 64-bit word");
  const int64_t s0 = span * kBwdSpan + (int64_t)wave * NT;
  if (s0 < L) {  // wave-uniform
    typename V::Raw xr[NXT], dr[NDT];
    const int32_t tl = (int32_t)(L - 1);
    // buffer loads: the row's byte offset is scalar (rows clamped into the
    // sequence), the lane's channels its 32-bit vector offset
    auto load_x = [&](int q) {
      const int32_t pos = (int32_t)s0 - (K - 1) + q;
      if (pos < 0 && sin)  // the carried-in window (the sequence's first tokens only)
        xr[q] = V::bload(rwin, loff, (uint32_t)(K - 1 + pos) * rowb);
      else
        xr[q] = V::bload(rx, loff, (uint32_t)(pos < 0 ? 0 : (pos < tl ? pos : tl)) * rowb);
    };
    auto load_d = [&](int j) {
      const int32_t pos = (int32_t)s0 + j;
      dr[j] = V::bload(rd, loff, (uint32_t)(pos < tl ? pos : tl) * rowb);
    };
    uint64_t starts = 0;  // bit q: a document starts at s0 - (K - 1) + q (real tokens only)
    if (p.reset) {
#pragma unroll
      for (int q = 0; q < NXT; ++q) {
        const int64_t pos = s0 - (K - 1) + q;
        if (pos >= 0 && pos < len && p.reset[b * L + pos]) starts |= 1ull << q;
      }
      // the same for every lane
      const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)starts);
      const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(starts >> 32));
      starts = (uint64_t)lo | ((uint64_t)hi << 32);
    }
    // no document starts at positions qa + 1 .. qb (window indices)
    auto visible = [&](int qa, int qb) -> bool {
      const uint64_t upto = qb >= 63 ? ~0ull : ((1ull << (qb + 1)) - 1ull);
      return (starts & upto & ~((1ull << (qa + 1)) - 1ull)) == 0;
    };
    // x at window index q, or 0 where the forward read a zero (before token 0
    // with no window given)
    auto xin = [&](int q, float (&o)[VEC]) {
      V::unpack(xr[q], o);
      if (s0 - (K - 1) + q < 0 && !sin) {
#pragma unroll
        for (int v = 0; v < VEC; ++v) o[v] = 0.0f;
      }
    };

    // the first kBwdT x positions (and the dout positions read with them); then
    // each position issues the loads kBwdT positions ahead (dout at j is first
    // read at x position j + K - 1)
#pragma unroll
    for (int q = 0; q < kBwdT; ++q) load_x(q);
#pragma unroll
    for (int j = 0; j < kBwdT - (K - 1); ++j) load_d(j);
    float xw[K][VEC], dpw[K][VEC];
#pragma unroll
    for (int i = 0; i < K; ++i)
#pragma unroll
      for (int v = 0; v < VEC; ++v) xw[i][v] = dpw[i][v] = 0.0f;
#pragma unroll
    for (int q = 0; q < NXT; ++q) {
      if (q + kBwdT < NXT) load_x(q + kBwdT);
      if (q + kBwdT - (K - 1) >= 0 && q + kBwdT - (K - 1) < NDT) load_d(q + kBwdT - (K - 1));
      // one position at a time: unpacking every loaded bf16 row at once would
      // hold them all as fp32, and the loads stay where they are issued
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = K - 1; i >= 1; --i)
#pragma unroll
        for (int v = 0; v < VEC; ++v) xw[i][v] = xw[i - 1][v];
      xin(q, xw[0]);
      if (q >= K - 1) {  // p = s0 + j
        const int j = q - (K - 1);
        const int64_t pp = s0 + j;
        float pre[VEC];
#pragma unroll
        for (int v = 0; v < VEC; ++v) pre[v] = bs[v];
#pragma unroll
        for (int i = 0; i < K; ++i) {
          const bool vis = visible(q - i, q);
#pragma unroll
          for (int v = 0; v < VEC; ++v) pre[v] = fmaf(wt[v][i], vis ? xw[i][v] : 0.0f, pre[v]);
        }
        float dov[VEC];
        V::unpack(dr[j], dov);
#pragma unroll
        for (int i = K - 1; i >= 1; --i)
#pragma unroll
          for (int v = 0; v < VEC; ++v) dpw[i][v] = dpw[i - 1][v];
#pragma unroll
        for (int v = 0; v < VEC; ++v) dpw[0][v] = pp < len ? dov[v] * act_prime(pre[v], silu) : 0.0f;
        if (j < NT && pp < len) {
#pragma unroll
          for (int i = 0; i < K; ++i) {
            const bool vis = visible(q - i, q);
#pragma unroll
            for (int v = 0; v < VEC; ++v) dw[v][i] = fmaf(dpw[0][v], vis ? xw[i][v] : 0.0f, dw[v][i]);
          }
#pragma unroll
          for (int v = 0; v < VEC; ++v) db[v] += dpw[0][v];
        }
      }
      if (q >= 2 * (K - 1)) {  // dx of s = s0 + m
        const int m = q - 2 * (K - 1);
        const int qs = q - (K - 1);
        const int64_t s = s0 + m;
        float acc[VEC];
#pragma unroll
        for (int v = 0; v < VEC; ++v) acc[v] = 0.0f;
#pragma unroll
        for (int i = 0; i < K; ++i) {  // dpre at s + i is dpw[K - 1 - i]
          const bool vis = visible(qs, qs + i);
#pragma unroll
          for (int v = 0; v < VEC; ++v) acc[v] = fmaf(wt[v][i], vis ? dpw[K - 1 - i][v] : 0.0f, acc[v]);
        }
        if (dso && s < len && s >= len - (K - 1) && visible(qs, (int)(len - 1 - s0) + K - 1)) {
          float o[VEC];
          dwo(s - (len - (K - 1)), o);
#pragma unroll
          for (int v = 0; v < VEC; ++v) acc[v] += o[v];
        }
        if (cok && s < L) V::store((IO*)p.dx + (b * L + s) * dim + c0, acc);
      }
      // the carried-in window's gradient, by the thread that starts the
      // sequence, once dpre at positions 0 .. K - 2 is known (dpre at P is
      // dpw[K - 2 - P])
      if (K > 1 && q == 2 * K - 3 && s0 == 0 && sin && p.dstate_in && cok) {
#pragma unroll
        for (int jw = 0; jw < K - 1; ++jw) {
          const int sw = -(K - 1) + jw;  // the window entry's position
          float acc[VEC];
#pragma unroll
          for (int v = 0; v < VEC; ++v) acc[v] = 0.0f;
#pragma unroll
          for (int i = 0; i < K; ++i) {
            if (sw + i >= 0) {
              const bool vis = visible(jw, jw + i);
#pragma unroll
              for (int v = 0; v < VEC; ++v)
                acc[v] = fmaf(wt[v][i], vis ? dpw[K - 2 - (sw + i)][v] : 0.0f, acc[v]);
            }
          }
          // a sequence shorter than the window hands on entries of this one
          if (dso && sw >= len - (K - 1) && (len == 0 || visible(jw, (int)(len - 1) + K - 1))) {
            float o[VEC];
            dwo(sw - (len - (K - 1)), o);
#pragma unroll
            for (int v = 0; v < VEC; ++v) acc[v] += o[v];
          }
          V::store((IO*)p.dstate_in + (b * (K - 1) + jw) * dim + c0, acc);
        }
      }
    }
  }

  // no tokens at all: the window passes through
  if (L == 0 && wave == 0 && sin && p.dstate_in && cok) {
#pragma unroll
    for (int j = 0; j < K - 1; ++j) {
      float o[VEC];
#pragma unroll
      for (int v = 0; v < VEC; ++v) o[v] = 0.0f;
      if (dso) dwo(j, o);
      V::store((IO*)p.dstate_in + (b * (K - 1) + j) * dim + c0, o);
    }
  }

  // ---- dw, dbias: the block's waves through LDS, one partial row per block
#pragma unroll
  for (int v = 0; v < VEC; ++v) {
#pragma unroll
    for (int i = 0; i < K; ++i) red[wave][v * (K + 1) + i][lane] = dw[v][i];
    red[wave][v * (K + 1) + K][lane] = db[v];
  }
  __syncthreads();
  if (wave == 0 && cok) {
    float* row = p.partial + (b * p.nspans + span) * (K + 1) * dim;
#pragma unroll
    for (int i = 0; i <= K; ++i) {
      float o[VEC];
#pragma unroll
      for (int v = 0; v < VEC; ++v) {
        float sum = 0.0f;
#pragma unroll
        for (int wv = 0; wv < kConvWaves; ++wv) sum += red[wv][v * (K + 1) + i][lane];
        o[v] = sum;
      }
      VecIO<float, VEC>::store(row + i * dim + c0, o);
    }
  }
}

// dw (dim, K) and dbias from the partial rows.  A block takes 32 consecutive
// sums; its 8 thread groups add every 8th row each (group g: rows g, g + 8,
// ...), and the 8 group sums are added in group order: a fixed order.
constexpr int kFinOut = 32, kFinGroups = 8;
__global__ __launch_bounds__(kFinOut * kFinGroups) void conv1d_bwd_finalize(
    const float* __restrict__ partial, float* __restrict__ dw, float* __restrict__ dbias,
    const int64_t rows, const int64_t dim, const int K) {
  __shared__ float part[kFinGroups][kFinOut];
  const int o = threadIdx.x % kFinOut, g = threadIdx.x / kFinOut;
  const int64_t e = (int64_t)blockIdx.x * kFinOut + o;  // (i, c) with i = e / dim
  const int64_t n = (int64_t)(K + 1) * dim;
  float sum = 0.0f;
  if (e < n) {
    const int i = (int)(e / dim);
    const int64_t c = e - (int64_t)i * dim;
    for (int64_t r = g; r < rows; r += kFinGroups) sum += partial[(r * (K + 1) + i) * dim + c];
  }
  part[g][o] = sum;
  __syncthreads();
  if (g == 0 && e < n) {
    float tot = 0.0f;
#pragma unroll
    for (int j = 0; j < kFinGroups; ++j) tot += part[j][o];
    const int i = (int)(e / dim);
    const int64_t c = e - (int64_t)i * dim;
    if (i < K) dw[c * K + i] = tot;
    else if (dbias) dbias[c] = tot;
  }
}

template <typename IO, int K, int VEC>
hipError_t bwd_launch(const ConvBwdParams& q, hipStream_t stream) {
  ConvBwdArgs a;
  a.x = q.x; a.state_in = q.state_in; a.dout = q.dout; a.dstate_out = q.dstate_out;
  a.w = q.w; a.bias = q.bias; a.seq_lens = q.seq_lens; a.reset = q.reset;
  a.dx = q.dx; a.dstate_in = q.dstate_in; a.partial = (float*)q.workspace;
  a.L = q.L; a.dim = q.dim; a.nspans = conv1d_bwd_spans(q.L); a.silu = q.silu;
  const int64_t nvec = q.dim / VEC;
  if (q.batch > 0) {  // no batch entries: the sums below are zero
    const dim3 grid((unsigned)((nvec + 63) / 64), (unsigned)a.nspans, (unsigned)q.batch);
    hipLaunchKernelGGL((conv1d_bwd_kernel<IO, K, VEC>), grid, dim3(64 * kConvWaves), 0, stream,
                       a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t n = (int64_t)(K + 1) * q.dim;
  hipLaunchKernelGGL(conv1d_bwd_finalize, dim3((unsigned)((n + kFinOut - 1) / kFinOut)),
                     dim3(kFinOut * kFinGroups), 0, stream, (const float*)a.partial, q.dw,
                     q.dbias, q.batch * a.nspans, q.dim, K);
  return hipGetLastError();
}

template <typename IO, int VEC>
hipError_t bwd_by_width(const ConvBwdParams& q, hipStream_t stream) {
  switch (q.k) {
    case 1: return bwd_launch<IO, 1, VEC>(q, stream);
    case 2: return bwd_launch<IO, 2, VEC>(q, stream);
    case 3: return bwd_launch<IO, 3, VEC>(q, stream);
    case 4: return bwd_launch<IO, 4, VEC>(q, stream);
    default: return hipErrorInvalidValue;
  }
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

int64_t conv1d_bwd_spans(int64_t L) { return L > 0 ? (L + kBwdSpan - 1) / kBwdSpan : 1; }

size_t conv1d_bwd_workspace_bytes(int64_t batch, int64_t L, int64_t dim, int64_t k) {
  return (size_t)batch * (size_t)conv1d_bwd_spans(L) * (size_t)(k + 1) * (size_t)dim * sizeof(float);
}

hipError_t launch_conv1d_bwd(const ConvBwdParams& q, int io_dtype, bool vec4, hipStream_t stream) {
  if (io_dtype == 1)
    return vec4 ? bwd_by_width<bf16_bits, 4>(q, stream) : bwd_by_width<bf16_bits, 1>(q, stream);
  return vec4 ? bwd_by_width<float, 4>(q, stream) : bwd_by_width<float, 1>(q, stream);
}

}  // namespace ssm66
