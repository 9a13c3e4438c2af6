// ssd.hip -- Mamba-2 / SSD layer (one scalar decay per head) on gfx950 MFMA.
//
// "Mamba and selective state spaces" (zerotofrontier.app/ssm/mamba), on what
// Mamba cannot do yet: giving each head (a group of P channels) a single
// scalar decay turns most of the work into matrix products; "State-space
// models & Mamba" (llm-tutorial.darvinyi.com), "The Mamba CUDA kernel": with
// the decay a scalar the layer is a structured masked matmul,
// Y = (M * (C B^T)) X, M[t, s] = exp(A sum_{s < r <= t} Delta_r), whose
// submatrices below the diagonal have rank one.  The recurrence per head:
//   h_t = exp(Delta_t A) h_{t-1} + w_t x_t B_t^T   (h: P x N per head),
//   y_t = h_t C_t + D x_t, gated by silu(z_t);  w = Delta (Euler) or
//   Delta phi(Delta A) (ZOH).
//
// Chunked form, Q = 64 tokens per chunk, cum_t the running sum of Delta A in
// the chunk:
//   Y     = exp(cum_t) (C H_in^T)  +  (C B^T * L) X,   L[t,s] = exp(cum_t - cum_s) w_s (t >= s)
//   H_out = exp(cum_Q) H_in + (exp(cum_Q - cum_s) w_s x_s)^T B.
// Every product is a dense contraction of bf16 operands with fp32
// accumulation on v_mfma_f32_16x16x32_bf16: lane l holds A[l%16][8(l/16)+j],
// B[8(l/16)+j][l%16] (j = 0..7) and D[4(l/16)+i][l%16] (i = 0..3).
//
// Work split: a block owns 16 of a head's 64 channels (one MFMA tile) for one
// batch entry and walks the chunks in order, so b * H * 4 blocks run at once
// (768 for 8 x 24 heads: three per CU).  The block recomputes the chunk's
// scores C B^T (they do not depend on the channel), and its 4 waves each take
// one 16-token row block of them, of Y, and a quarter of the state's columns,
// which stay in MFMA accumulators (fp32) for the whole sequence.
//
// Orientation: products that contract over tokens need operands with tokens
// contiguous; x and B arrive token-major, so those operands are read with
// ds_read_b64_tr_b16 (a transposing LDS read) from row-major copies.  The
// scores are formed transposed (S^T tiles from B C^T) and the state as H^T, so
// each lane's four results are consecutive in the row-major layout the next
// product reads, and every LDS write is 8 bytes; Y comes out as Y^T, four
// consecutive channels of one token per lane, stored as 8 bytes.  C never
// enters LDS: each wave reads the 16 C rows of its token block straight into
// the operand registers (the same fragment serves C B^T and H C^T).
//
// Only P = 64 and N in {64, 128} with bf16 io are instantiated.
#include "ssm_device.h"
#include "ssm_launch.h"

namespace ssm66 {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(8))) short i16x8;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kQ = 64;               // tokens per chunk
constexpr int kP = 64;               // channels per head
constexpr int kPS = 16;              // channels per block
constexpr int kSlices = kP / kPS;    // blocks per (batch entry, head)
constexpr int kWaves = 4;

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ float lo_bf(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float hi_bf(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// The MFMA operand fragment "row r = l % 16, k = 8 (l / 16) + j" of a matrix
// stored k-major in LDS (element (k, r) at base[k * STRIDE + r]), i.e. the
// transpose of what a row read gives.  ds_read_b64_tr_b16 works on groups of
// 16 lanes: lane i receives, as its 4 values k = 0..3, element i % 4 of the
// 8 bytes addressed by lane 4 k + i / 4 of its group.  So lane (g, kk, qq) =
// (l / 16, (l % 16) / 4, l % 4) addresses row 8 g + kk (+ 4 in the second
// read), columns 4 qq .. 4 qq + 3.
template <int STRIDE>
__device__ __forceinline__ bf16x8 tr_frag(const __bf16* base, int lane) {
  const int g = lane >> 4, kk = (lane & 15) >> 2, qq = lane & 3;
  const __bf16* p0 = base + (8 * g + kk) * STRIDE + 4 * qq;
  const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(void*)p0);
  const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(void*)(p0 + 4 * STRIDE));
  const i16x8 v = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// Row strides (bf16 elements).  Bs and Hs rows are read 16 bytes per lane,
// rows l % 16: a stride of 4 dwords mod 32 puts 8 consecutive rows on distinct
// banks.  Xs rows are 32 bytes, so the 16 lanes of a transposing read (4 rows
// x 4 column quads) cover the 32 banks once.
template <int N>
struct alignas(16) SSDSmem {
  static constexpr int BS = N + 8;
  static constexpr int SS = kQ + 8;
  __bf16 Bs[kQ][BS];            // B rows of the chunk (n contiguous)
  __bf16 Xs[kQ][kPS];           // this block's x columns (p contiguous)
  __bf16 Ss[kQ][SS];            // masked scores S[t][s] (s contiguous)
  __bf16 Hs[2][kPS][BS];        // the state entering the chunk, bf16, double-buffered
  float cuml[kQ];               // running sum of Delta A in the chunk, times log2 e
  float wv[kQ];                 // input weight w_s
  float eend[kQ];               // exp(cum_Q - cum_s) w_s
  float et[kQ];                 // exp(cum_t)
};

struct SSDArgs {
  const bf16_bits *x, *B, *C, *z;
  const float *dt, *A, *D, *dt_bias, *h0;
  bf16_bits* y;
  float* last_state;
  int64_t batch, L, nheads;
  int softplus;
};

template <int N, bool ZOH, bool GATE>
__global__ __launch_bounds__(256, 3) void ssd_fwd_kernel(const SSDArgs p) {
  using Sm = SSDSmem<N>;
  __shared__ Sm sm;
  constexpr int NK = N / 32;               // k-steps over the states
  constexpr int NTW = N / 16 / kWaves;     // state column tiles per wave
  constexpr int RB = kQ * N / 8 / 256;     // 16-byte pieces of B per thread
  static_assert(NTW >= 1 && RB >= 1, "N is 64 or 128");
  const int64_t H = p.nheads, L = p.L, HP = H * kP;

  // XCD-aware order: consecutive block ids go round-robin to the 8 XCDs, so
  // each XCD gets a contiguous run of (batch entry, head, slice) -- the blocks
  // of one batch entry share its B and C rows in that XCD's L2.
  const int64_t nblk = (int64_t)gridDim.x, bid = blockIdx.x;
  const int64_t logical = (nblk % 8 == 0) ? (bid % 8) * (nblk / 8) + bid / 8 : bid;
  const int64_t bh = logical / kSlices;
  const int q = (int)(logical - bh * kSlices);
  const int64_t b = bh / H, h = bh - b * H;
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;   // wave w: token block 16 w .. 16 w + 15
  const int lr = lane & 15, lk = lane >> 4;  // MFMA row / k-group of this lane
  const float A = p.A[h];
  const float Dh = p.D ? p.D[h] : 0.0f;
  const float bias = p.dt_bias ? p.dt_bias[h] : 0.0f;
  const int64_t ch0 = h * kP + q * kPS;      // first channel of the block in a row of x, z, y

  // ---- the state, as H^T tiles: wave w holds column tiles nt = w + 4 j;
  // lane value i is H[p = lr][n = 16 nt + 4 lk + i]
  const int64_t hrow = ((b * H + h) * kP + q * kPS + lr) * N;
  f32x4 Hacc[NTW];
#pragma unroll
  for (int j = 0; j < NTW; ++j) {
    const int n = 16 * (w + kWaves * j) + 4 * lk;
    Hacc[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    if (p.h0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) Hacc[j][i] = p.h0[hrow + n + i];
    }
    *(u32x2*)&sm.Hs[0][lr][n] =
        u32x2{pack_bf16x2(Hacc[j][0], Hacc[j][1]), pack_bf16x2(Hacc[j][2], Hacc[j][3])};
  }

  // ---- global reads of one chunk into registers; rows past L are clamped to
  // the last row (finite data that the zero weights of padding tokens cancel).
  // Issued for the next chunk before this chunk's products.
  u32x4 rB[RB], rC[NK];
  u32x2 rX, rZ = u32x2{0u, 0u};
  float rdt;
  auto load_chunk = [&](int64_t t0) {
    const int64_t last = L - 1;
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int e = tid + 256 * r;
      const int s = e / (N / 8), c8 = (e % (N / 8)) * 8;
      const int64_t row = b * L + (t0 + s < L ? t0 + s : last);
      rB[r] = *(const u32x4*)(p.B + row * N + c8);
    }
    {  // C rows of this wave's token block; z of this lane's output
      const int64_t t = t0 + 16 * w + lr;
      const int64_t row = b * L + (t < L ? t : last);
#pragma unroll
      for (int k = 0; k < NK; ++k) rC[k] = *(const u32x4*)(p.C + row * N + 32 * k + 8 * lk);
      if constexpr (GATE) rZ = *(const u32x2*)(p.z + row * HP + ch0 + 4 * lk);
    }
    {  // x: token tid / 4, channels 4 (tid % 4) ..
      const int64_t t = t0 + (tid >> 2);
      const int64_t row = b * L + (t < L ? t : last);
      rX = *(const u32x2*)(p.x + row * HP + ch0 + 4 * (tid & 3));
    }
    {
      const int64_t t = t0 + lane;
      rdt = p.dt[(b * L + (t < L ? t : last)) * H + h];
    }
  };

  const int64_t nchunks = (L + kQ - 1) / kQ;
  if (nchunks > 0) load_chunk(0);
  for (int64_t ck = 0; ck < nchunks; ++ck) {
    const int64_t t0 = ck * kQ;
    const int nlive = (int)(L - t0 < kQ ? L - t0 : kQ);
    const int cur = (int)(ck & 1);

    // ---- stage B rows and the x columns (x rows past L as zeros)
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int e = tid + 256 * r;
      *(u32x4*)&sm.Bs[e / (N / 8)][(e % (N / 8)) * 8] = rB[r];
    }
    *(u32x2*)&sm.Xs[tid >> 2][4 * (tid & 3)] = (tid >> 2) < nlive ? rX : u32x2{0u, 0u};
    u32x4 cC[NK];
#pragma unroll
    for (int k = 0; k < NK; ++k) cC[k] = rC[k];
    const u32x2 cZ = rZ;
    const float raw = rdt;
    if (ck + 1 < nchunks) load_chunk(t0 + kQ);

    // ---- step sizes, decays and weights of the chunk (wave 0, lane = token)
    if (w == 0) {
      const float v = raw + bias;
      float dl = p.softplus ? softplus_f(v) : v;
      if (lane >= nlive) dl = 0.0f;  // padding: no decay, no input
      const float a = dl * A;
      float wt = dl;
      if constexpr (ZOH) wt = dl * zoh_phi(a, exp2_hw(a * kLog2e));
      float c = a * kLog2e;  // inclusive running sum, log2 units
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float o = __shfl_up(c, off, 64);
        if (lane >= off) c += o;
      }
      const float cend = __shfl(c, 63, 64);
      sm.cuml[lane] = c;
      sm.wv[lane] = wt;
      sm.eend[lane] = exp2_hw(cend - c) * wt;
      sm.et[lane] = exp2_hw(c);
    }
    lds_barrier();

    // ---- scores of this wave's token block t = 16 w .. : S^T tiles
    // D[s][t] = sum_n B[s][n] C[t][n], masked to S[t][s] = D exp(cum_t - cum_s) w_s
    // (s <= t); lane value i is s = 16 sb + 4 lk + i, t = 16 w + lr
    {
      const float ct = sm.cuml[16 * w + lr];
#pragma unroll
      for (int sb = 0; sb < 4; ++sb) {
        if (sb <= w) {
          f32x4 g = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int k = 0; k < NK; ++k)
            g = mfma16(*(const bf16x8*)&sm.Bs[16 * sb + lr][32 * k + 8 * lk], as_bf16x8(cC[k]), g);
          const float4 cs = *(const float4*)&sm.cuml[16 * sb + 4 * lk];
          const float4 ws = *(const float4*)&sm.wv[16 * sb + 4 * lk];
          const float csv[4] = {cs.x, cs.y, cs.z, cs.w}, wsv[4] = {ws.x, ws.y, ws.z, ws.w};
          float v[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const bool keep = sb < w || 4 * lk + i <= lr;  // s <= t
            v[i] = keep ? g[i] * exp2_hw(ct - csv[i]) * wsv[i] : 0.0f;
          }
          *(u32x2*)&sm.Ss[16 * w + lr][16 * sb + 4 * lk] =
              u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        } else if (sb == w + 1 && (w & 1) == 0) {
          // the tile past the diagonal that the 32-wide k-steps of S X read
          *(u32x2*)&sm.Ss[16 * w + lr][16 * sb + 4 * lk] = u32x2{0u, 0u};
        }
      }
    }
    lds_barrier();

    // ---- Y^T for token block w: D[p][t] = exp(cum_t) sum_n H[p][n] C[t][n]
    //      + sum_s x[s][p] S[t][s]; lane value i is p = 4 lk + i, t = 16 w + lr
    {
      f32x4 y = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int k = 0; k < NK; ++k)
        y = mfma16(*(const bf16x8*)&sm.Hs[cur][lr][32 * k + 8 * lk], as_bf16x8(cC[k]), y);
      const float e = sm.et[16 * w + lr];
#pragma unroll
      for (int i = 0; i < 4; ++i) y[i] *= e;
#pragma unroll
      for (int s0 = 0; s0 < kQ; s0 += 32) {
        if (s0 <= 16 * w + 15) {  // scores past the diagonal block are zero
          const bf16x8 xa = tr_frag<kPS>(&sm.Xs[s0][0], lane);
          y = mfma16(xa, *(const bf16x8*)&sm.Ss[16 * w + lr][s0 + 8 * lk], y);
        }
      }
      // ---- epilogue: skip, gate, store 4 channels of token t
      const int t = 16 * w + lr;
      if (t < nlive) {
        const u32x2 xv = *(const u32x2*)&sm.Xs[t][4 * lk];
        float o[4] = {fmaf(Dh, lo_bf(xv.x), y[0]), fmaf(Dh, hi_bf(xv.x), y[1]),
                      fmaf(Dh, lo_bf(xv.y), y[2]), fmaf(Dh, hi_bf(xv.y), y[3])};
        if constexpr (GATE) {
          o[0] *= silu_f(lo_bf(cZ.x));
          o[1] *= silu_f(hi_bf(cZ.x));
          o[2] *= silu_f(lo_bf(cZ.y));
          o[3] *= silu_f(hi_bf(cZ.y));
        }
        *(u32x2*)(p.y + (b * L + t0 + t) * HP + ch0 + 4 * lk) =
            u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
      }
    }

    // ---- state update, H^T tiles: D[n][p] = exp(cum_Q) H^T[n][p]
    //      + sum_s B[s][n] (eend_s x[s][p])
    {
      const float etot = exp2_hw(sm.cuml[kQ - 1]);
#pragma unroll
      for (int j = 0; j < NTW; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) Hacc[j][i] *= etot;
#pragma unroll
      for (int s0 = 0; s0 < kQ; s0 += 32) {
        const bf16x8 xt = tr_frag<kPS>(&sm.Xs[s0][0], lane);  // x[s0 + 8 lk + j][lr]
        const float4 e0 = *(const float4*)&sm.eend[s0 + 8 * lk];
        const float4 e1 = *(const float4*)&sm.eend[s0 + 8 * lk + 4];
        const float ev[8] = {e0.x, e0.y, e0.z, e0.w, e1.x, e1.y, e1.z, e1.w};
        bf16x8 xw;
#pragma unroll
        for (int j = 0; j < 8; ++j) xw[j] = (__bf16)((float)xt[j] * ev[j]);
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
          const bf16x8 bt = tr_frag<Sm::BS>(&sm.Bs[s0][16 * (w + kWaves * j)], lane);
          Hacc[j] = mfma16(bt, xw, Hacc[j]);
        }
      }
      const int nxt = cur ^ 1;  // last read in the previous chunk, before its barriers
#pragma unroll
      for (int j = 0; j < NTW; ++j)
        *(u32x2*)&sm.Hs[nxt][lr][16 * (w + kWaves * j) + 4 * lk] =
            u32x2{pack_bf16x2(Hacc[j][0], Hacc[j][1]), pack_bf16x2(Hacc[j][2], Hacc[j][3])};
    }
    lds_barrier();  // every wave is done with Bs, Xs, Ss and the chunk's constants
  }

  if (p.last_state) {
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
      const int n = 16 * (w + kWaves * j) + 4 * lk;
#pragma unroll
      for (int i = 0; i < 4; ++i) p.last_state[hrow + n + i] = Hacc[j][i];
    }
  }
}

template <int N, bool ZOH, bool GATE>
hipError_t ssd_launch(const SSDArgs& a, hipStream_t stream) {
  const int64_t nblk = a.batch * a.nheads * kSlices;
  if (nblk > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((ssd_fwd_kernel<N, ZOH, GATE>), dim3((unsigned)nblk), dim3(64 * kWaves), 0,
                     stream, a);
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
  if (q.P != kP) return hipErrorInvalidValue;
  if (q.N == 128) return ssd_modes<128>(a, zoh, gate, stream);
  if (q.N == 64) return ssd_modes<64>(a, zoh, gate, stream);
  return hipErrorInvalidValue;
}

}  // namespace ssm66
