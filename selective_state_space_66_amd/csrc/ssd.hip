// ssd.hip -- Mamba-2 / SSD layer (one scalar decay per head) on gfx950 MFMA.
//
// "Mamba and selective state spaces" (zerotofrontier.app/ssm/mamba), on what
// Mamba cannot do yet: giving each head (a group of P channels) a single
// scalar decay turns most of the work into matrix products; "State-space
// models & Mamba" (llm-tutorial.darvinyi.com), "The Mamba CUDA kernel": with
// the decay a scalar the layer is a structured masked matmul,
// Y = (M * (C B^T)) X, M[t, s] = exp(A sum_{s < r <= t} Delta_r), whose
// submatrices below the diagonal have rank one.  The recurrence per head:
//   h_t = exp(Delta_t A) h_{t-1} + w_t B_t x_t^T   (h: P x N per head),
//   y_t = h_t C_t + D x_t, gated by silu(z_t);  w = Delta (Euler) or
//   Delta phi(Delta A) (ZOH).
//
// Chunked form, Q = 64 tokens per chunk, cum_t the running sum of Delta A in
// the chunk:
//   Y     = exp(cum_t) (C H_in^T)  +  (C B^T * L) X,   L[t,s] = exp(cum_t - cum_s) w_s (t >= s)
//   H_out = exp(cum_Q) H_in + (exp(cum_Q - cum_s) w_s x_s)^T B.
// Every product is a dense contraction of bf16 operands with fp32
// accumulation: v_mfma_f32_16x16x32_bf16 (lane l holds A[l%16][8(l/16)+j],
// B[8(l/16)+j][l%16] and D[4(l/16)+i][l%16]).
//
// A block owns one (batch entry, head) and walks its chunks in order; its 4
// waves split each product by 16-row blocks, and the head's P x N state stays
// in the waves' MFMA accumulators (fp32) for the whole sequence -- nothing is
// written between chunks.  Operands are staged in LDS in the orientation each
// product reads with 16-byte loads (B row-major for C B^T, B transposed for the
// state update, x transposed).  Only P = 64 and N in {64, 128} with bf16 io
// are instantiated.
#include "ssm_device.h"
#include "ssm_launch.h"

namespace ssm66 {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
// 16 bytes as a native vector (HIP's uint4 is a class around a union, which
// can keep arrays of it out of registers)
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

constexpr int kQ = 64;   // tokens per chunk
constexpr int kP = 64;   // channels per head
constexpr int kPad = 8;  // row padding (bf16) against LDS bank conflicts

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ __bf16 to_bf(float v) { return (__bf16)v; }
// a 16-byte load seen as 8 bf16 values (a bit cast: no address is taken, so
// the value stays in registers)
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ float from_bf(__bf16 v) { return (float)v; }

template <int N>
struct SSDSmem {
  __bf16 Bs[kQ][N + kPad];    // B rows: n contiguous
  __bf16 Bt[N][kQ + kPad];    // B transposed: s contiguous
  __bf16 Cs[kQ][N + kPad];
  __bf16 Xt[kP][kQ + kPad];   // x transposed: t contiguous
  __bf16 Ss[kQ][kQ + kPad];   // masked scores
  __bf16 Hs[kP][N + kPad];    // the state entering the chunk, bf16
  __bf16 Zs[kQ][kP + kPad];   // gate input rows
  float cum[kQ], wv[kQ], eend[kQ], et[kQ];
};

struct SSDArgs {
  const bf16_bits *x, *B, *C, *z;
  const float *dt, *A, *D, *dt_bias, *h0;
  bf16_bits* y;
  float* last_state;
  int64_t batch, L, nheads;
  int softplus;
};

// Global reads of one chunk into registers: clamped rows (rows past L are
// zeroed when written to LDS).  Issued for the next chunk before this chunk's
// products, so they land while those run.
template <int N, bool GATE>
__device__ __forceinline__ void ssd_load_chunk(const SSDArgs& p, int64_t b, int64_t h, int64_t t0,
                                               int tid, u32x4 (&rB)[kQ * N / 8 / 256],
                                               u32x4 (&rC)[kQ * N / 8 / 256],
                                               u32x4 (&rX)[kQ * kP / 8 / 256],
                                               u32x4 (&rZ)[kQ * kP / 8 / 256], float& rdt) {
  const int64_t L = p.L, H = p.nheads, HP = H * kP, last = L - 1;
#pragma unroll
  for (int r = 0; r < kQ * N / 8 / 256; ++r) {
    const int e = tid + 256 * r;
    const int s = e / (N / 8), c8 = (e % (N / 8)) * 8;
    const int64_t row = b * L + (t0 + s < L ? t0 + s : last);
    rB[r] = *(const u32x4*)(p.B + row * N + c8);
    rC[r] = *(const u32x4*)(p.C + row * N + c8);
  }
#pragma unroll
  for (int r = 0; r < kQ * kP / 8 / 256; ++r) {
    const int e = tid + 256 * r;
    const int s = e / (kP / 8), c8 = (e % (kP / 8)) * 8;
    const int64_t row = b * L + (t0 + s < L ? t0 + s : last);
    rX[r] = *(const u32x4*)(p.x + row * HP + h * kP + c8);
    if constexpr (GATE) rZ[r] = *(const u32x4*)(p.z + row * HP + h * kP + c8);
  }
  const int lane = tid & 63;
  if (tid < 64) rdt = p.dt[(b * L + (t0 + lane < L ? t0 + lane : last)) * H + h];
}

template <int N, bool ZOH, bool GATE>
__global__ __launch_bounds__(256) void ssd_fwd_kernel(const SSDArgs p) {
  __shared__ SSDSmem<N> sm;
  constexpr int NT = N / 16;  // 16-column tiles of the state
  const int64_t H = p.nheads, L = p.L, HP = H * kP;
  const int64_t bh = blockIdx.x;
  const int64_t b = bh / H, h = bh - b * H;
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;  // wave = 16-row block
  const int lr = lane & 15, lk = lane >> 4;  // MFMA row / k-group of this lane
  const float A = p.A[h];
  const float Dh = p.D ? p.D[h] : 0.0f;
  const float bias = p.dt_bias ? p.dt_bias[h] : 0.0f;

  // ---- the state: rows p = 16 w + 4 lk + i, columns n = 16 nt + lr
  f32x4 Hacc[NT];
  if (p.h0) {  // one uniform branch: all loads in flight together
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        Hacc[nt][i] = p.h0[((b * H + h) * kP + 16 * w + 4 * lk + i) * N + 16 * nt + lr];
  } else {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) Hacc[nt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int i = 0; i < 4; ++i) sm.Hs[16 * w + 4 * lk + i][16 * nt + lr] = to_bf(Hacc[nt][i]);

  // ---- global reads of one chunk into registers (clamped rows; rows past L
  // are zeroed when they are written to LDS).  The next chunk's reads are
  // issued before this chunk's products, so they land while those run.
  constexpr int RB = kQ * N / 8 / 256;   // 16-byte pieces of B (and of C) per thread
  constexpr int RX = kQ * kP / 8 / 256;  // of x (and of z)
  u32x4 rB[RB], rC[RB], rX[RX], rZ[RX];
  float rdt = 0.0f;
  const int64_t nchunks = (L + kQ - 1) / kQ;
  if (nchunks > 0) ssd_load_chunk<N, GATE>(p, b, h, 0, tid, rB, rC, rX, rZ, rdt);
  for (int64_t ck = 0; ck < nchunks; ++ck) {
    const int64_t t0 = ck * kQ;
    const int nt_live = (int)(L - t0 < kQ ? L - t0 : kQ);
    // ---- stage the chunk's B, C, x, z (rows past L as zeros)
    const u32x4 zero4 = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int e = tid + 256 * r;
      const int s = e / (N / 8), c8 = (e % (N / 8)) * 8;
      const bool live = s < nt_live;
      const u32x4 vb = live ? rB[r] : zero4;
      *(u32x4*)&sm.Bs[s][c8] = vb;
      *(u32x4*)&sm.Cs[s][c8] = live ? rC[r] : zero4;
      const bf16x8 pb = as_bf16x8(vb);
#pragma unroll
      for (int j = 0; j < 8; ++j) sm.Bt[c8 + j][s] = pb[j];
    }
#pragma unroll
    for (int r = 0; r < RX; ++r) {
      const int e = tid + 256 * r;
      const int s = e / (kP / 8), c8 = (e % (kP / 8)) * 8;
      const bool live = s < nt_live;
      const u32x4 vx = live ? rX[r] : zero4;
      const bf16x8 px = as_bf16x8(vx);
#pragma unroll
      for (int j = 0; j < 8; ++j) sm.Xt[c8 + j][s] = px[j];
      if constexpr (GATE) *(u32x4*)&sm.Zs[s][c8] = live ? rZ[r] : zero4;
    }
    const float raw = rdt;
    if (ck + 1 < nchunks) ssd_load_chunk<N, GATE>(p, b, h, t0 + kQ, tid, rB, rC, rX, rZ, rdt);
    // ---- step sizes, decays and weights of the chunk (wave 0)
    if (w == 0) {
      const int s = lane;
      const bool live = s < nt_live;
      const float v = raw + bias;
      float dl = p.softplus ? softplus_f(v) : v;
      if (!live) dl = 0.0f;  // padding: no decay, no write
      const float a = dl * A;
      float wt = dl;
      if constexpr (ZOH) wt = dl * zoh_phi(a, exp2_hw(a * kLog2e));
      // inclusive running sum of a over the 64 tokens
      float cum = a;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float o = __shfl_up(cum, off, 64);
        if (lane >= off) cum += o;
      }
      const float cend = __shfl(cum, 63, 64);
      sm.cum[s] = cum;
      sm.wv[s] = wt;
      sm.eend[s] = exp2_hw((cend - cum) * kLog2e) * wt;
      sm.et[s] = exp2_hw(cum * kLog2e);
    }
    lds_barrier();

    // ---- masked scores S = (C B^T) * L for rows 16 w .. 16 w + 15
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      f32x4 g = {0.0f, 0.0f, 0.0f, 0.0f};
      if (ct <= w) {
#pragma unroll 2
        for (int k0 = 0; k0 < N; k0 += 32) {
          const bf16x8 a = *(const bf16x8*)&sm.Cs[16 * w + lr][k0 + 8 * lk];
          const bf16x8 bb = *(const bf16x8*)&sm.Bs[16 * ct + lr][k0 + 8 * lk];
          g = mfma16(a, bb, g);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * w + 4 * lk + i, s = 16 * ct + lr;
        float val = 0.0f;
        if (ct <= w && t >= s) val = g[i] * exp2_hw((sm.cum[t] - sm.cum[s]) * kLog2e) * sm.wv[s];
        sm.Ss[t][s] = to_bf(val);
      }
    }
    lds_barrier();

    // ---- Y = exp(cum_t) (C H_in^T) + S X, rows 16 w .., columns 16 pt ..
    f32x4 Y[4];
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) Y[pt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 1
    for (int k0 = 0; k0 < N; k0 += 32) {
      const bf16x8 a = *(const bf16x8*)&sm.Cs[16 * w + lr][k0 + 8 * lk];
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        const bf16x8 bb = *(const bf16x8*)&sm.Hs[16 * pt + lr][k0 + 8 * lk];
        Y[pt] = mfma16(a, bb, Y[pt]);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float e = sm.et[16 * w + 4 * lk + i];
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) Y[pt][i] *= e;
    }
#pragma unroll
    for (int k0 = 0; k0 < kQ; k0 += 32) {
      if (k0 <= 16 * w + 15) {  // scores past the diagonal block are zero
        const bf16x8 a = *(const bf16x8*)&sm.Ss[16 * w + lr][k0 + 8 * lk];
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
          const bf16x8 bb = *(const bf16x8*)&sm.Xt[16 * pt + lr][k0 + 8 * lk];
          Y[pt] = mfma16(a, bb, Y[pt]);
        }
      }
    }
    // ---- epilogue: skip, gate, store
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * w + 4 * lk + i, pc = 16 * pt + lr;
        if (t < nt_live) {
          const float xv = from_bf(sm.Xt[pc][t]);
          float out = fmaf(Dh, xv, Y[pt][i]);
          const int64_t yi = (b * L + t0 + t) * HP + h * kP + pc;
          if constexpr (GATE) out *= silu_f(from_bf(sm.Zs[t][pc]));
          store_io(p.y + yi, out);
        }
      }
    }

    // ---- state update: H = exp(cum_Q) H + (eend x)^T B, rows p = 16 w ..
    const float etot = exp2_hw(sm.cum[kQ - 1] * kLog2e);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) Hacc[nt][i] *= etot;
#pragma unroll 1
    for (int k0 = 0; k0 < kQ; k0 += 32) {
      const bf16x8 xr = *(const bf16x8*)&sm.Xt[16 * w + lr][k0 + 8 * lk];
      bf16x8 a;
#pragma unroll
      for (int j = 0; j < 8; ++j) a[j] = to_bf(from_bf(xr[j]) * sm.eend[k0 + 8 * lk + j]);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const bf16x8 bb = *(const bf16x8*)&sm.Bt[16 * nt + lr][k0 + 8 * lk];
        Hacc[nt] = mfma16(a, bb, Hacc[nt]);
      }
    }
    lds_barrier();  // every wave is done with Hs, Bs, Bt, Cs, Xt, Ss of this chunk
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.Hs[16 * w + 4 * lk + i][16 * nt + lr] = to_bf(Hacc[nt][i]);
    // the next chunk's staging writes other arrays; its first barrier orders Hs
  }

  if (p.last_state) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int pp = 16 * w + 4 * lk + i, n = 16 * nt + lr;
        p.last_state[((b * H + h) * kP + pp) * N + n] = Hacc[nt][i];
      }
  }
}

template <int N, bool ZOH, bool GATE>
hipError_t ssd_launch(const SSDArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((ssd_fwd_kernel<N, ZOH, GATE>), dim3((unsigned)(a.batch * a.nheads)),
                     dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int N>
hipError_t ssd_modes(const SSDArgs& a, bool zoh, bool gate, hipStream_t stream) {
  if (zoh) return gate ? ssd_launch<N, true, true>(a, stream) : ssd_launch<N, true, false>(a, stream);
  return gate ? ssd_launch<N, false, true>(a, stream) : ssd_launch<N, false, false>(a, stream);
}

}  // namespace

hipError_t launch_ssd_fwd(const SSDParams& q, bool zoh, bool gate, hipStream_t stream) {
  SSDArgs a;
  a.x = (const bf16_bits*)q.x; a.B = (const bf16_bits*)q.B; a.C = (const bf16_bits*)q.C;
  a.z = (const bf16_bits*)q.z; a.dt = q.dt; a.A = q.A; a.D = q.D; a.dt_bias = q.dt_bias;
  a.h0 = q.h0; a.y = (bf16_bits*)q.y; a.last_state = q.last_state;
  a.batch = q.batch; a.L = q.L; a.nheads = q.nheads; a.softplus = q.softplus;
  if (q.N == 128) return ssd_modes<128>(a, zoh, gate, stream);
  if (q.N == 64) return ssd_modes<64>(a, zoh, gate, stream);
  return hipErrorInvalidValue;
}

}  // namespace ssm66
