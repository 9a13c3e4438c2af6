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

// Per-token constants of one chunk, from its step sizes.
struct ChunkConsts {
  float cuml[kQ];   // running sum of Delta A in the chunk, times log2 e
  float wv[kQ];     // input weight w_s
  float fw[kQ];     // exp(cum* - cum_s) w_s, cum* = cum at the end of s's 16-block
  float eend[kQ];   // exp(cum_Q - cum_s) w_s
  float et[kQ];     // exp(cum_t)
};

// The K = 16 MFMA (v_mfma_f32_16x16x16_bf16): lane l holds A[l%16][4(l/16)+j]
// and B[4(l/16)+j][l%16], j = 0..3; D as for K = 32.
__device__ __forceinline__ f32x4 mfma16k16(i16x4 a, i16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// The K = 16 operand fragment "row r = l % 16, k = 4 (l / 16) + j" of a
// matrix stored k-major in LDS: one transposing read, lane (g, kk, qq)
// addressing row 4 g + kk, columns 4 qq .. 4 qq + 3.
template <int STRIDE>
__device__ __forceinline__ i16x4 tr_frag4(const __bf16* base, int lane) {
  const int g = lane >> 4, kk = (lane & 15) >> 2, qq = lane & 3;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)(void*)(base + (4 * g + kk) * STRIDE + 4 * qq));
}

// Row strides (bf16 elements).  Bs and Hs rows are read 16 bytes per lane,
// rows l % 16: a stride of 4 dwords mod 32 puts 8 consecutive rows on distinct
// banks.  Xs rows are 32 bytes, so the 16 lanes of a transposing read (4 rows
// x 4 column quads) cover the 32 banks once.  Everything a chunk reads is
// double-buffered by chunk parity, so staging the next chunk does not wait for
// the current one: one barrier per chunk.
template <int N>
struct alignas(16) SSDSmem {
  static constexpr int BS = N + 8;
  __bf16 Bs[2][kQ][BS];         // B rows of a chunk (n contiguous)
  __bf16 Xs[2][kQ][kPS];        // this block's x columns (p contiguous)
  __bf16 Hs[2][kPS][BS];        // the state entering a chunk, bf16
  ChunkConsts cc[2];            // per-token constants
};

struct SSDArgs {
  const bf16_bits *x, *B, *C, *z;
  const float *dt, *A, *D, *dt_bias, *h0;
  bf16_bits* y;
  float* last_state;
  int64_t batch, L, nheads;
  int softplus;
};

// Inclusive prefix sum over the 64 lanes of a wave with DPP: shifts of 1, 2,
// 4 and 8 lanes inside each row of 16 (lanes shifted in from outside the row
// add 0), then the last lane of row 0 and 2 added to rows 1 and 3, and lane 31
// added to rows 2 and 3.
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_or_zero(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWS, 0xf, true));
}
__device__ __forceinline__ float wave_inclusive_sum(float v) {
  v += dpp_or_zero<0x111, 0xf>(v);  // row_shr:1
  v += dpp_or_zero<0x112, 0xf>(v);  // row_shr:2
  v += dpp_or_zero<0x114, 0xf>(v);  // row_shr:4
  v += dpp_or_zero<0x118, 0xf>(v);  // row_shr:8
  v += dpp_or_zero<0x142, 0xa>(v);  // row_bcast:15 into rows 1, 3
  v += dpp_or_zero<0x143, 0xc>(v);  // row_bcast:31 into rows 2, 3
  return v;
}

__device__ __forceinline__ float lane_value(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// The scores of token block W and their product with x (waves are specialised
// on W: all branches on it are uniform).  S^T tiles D[s][t] = sum_n B[s][n]
// C[t][n] for the s blocks sb <= W (the tiles' MFMA chains interleaved) are
// masked and weighted to S[t][s] = D exp(cum_t - cum_s) w_s (s <= t).  Below
// the diagonal block the decay factors through the end of block sb, cum*:
// exp(cum_t - cum*) exp(cum* - cum_s) w_s, both factors at most 1, the second
// one per token (fw) -- one exponential per lane and tile; on the diagonal
// block it is taken directly.  A tile's lane values (s = 16 sb + 4 lk + i,
// t = 16 W + lr) are, rounded to bf16, exactly the B operand of the K = 16
// MFMA (4 consecutive k per lane), so Y^T += x^T S^T takes them from registers.
template <int W, int N, class Sm>
__device__ __forceinline__ void scores_times_x(const Sm& sm, int cur, const ChunkConsts& kc,
                                               const u32x4 (&cC)[N / 32], int lane, f32x4& y) {
  const int lr = lane & 15, lk = lane >> 4;
  f32x4 g[W + 1];
#pragma unroll
  for (int sb = 0; sb <= W; ++sb) g[sb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int k = 0; k < N / 32; ++k)
#pragma unroll
    for (int sb = 0; sb <= W; ++sb)
      g[sb] = mfma16(*(const bf16x8*)&sm.Bs[cur][16 * sb + lr][32 * k + 8 * lk], as_bf16x8(cC[k]),
                     g[sb]);
  const float ct = kc.cuml[16 * W + lr];
#pragma unroll
  for (int sb = 0; sb <= W; ++sb) {
    float v[4];
    if (sb < W) {
      const float gt = exp2_hw(ct - kc.cuml[16 * sb + 15]);
      const float4 fw = *(const float4*)&kc.fw[16 * sb + 4 * lk];
      v[0] = g[sb][0] * fw.x * gt;
      v[1] = g[sb][1] * fw.y * gt;
      v[2] = g[sb][2] * fw.z * gt;
      v[3] = g[sb][3] * fw.w * gt;
    } else {
      const float4 cs = *(const float4*)&kc.cuml[16 * sb + 4 * lk];
      const float4 ws = *(const float4*)&kc.wv[16 * sb + 4 * lk];
      const float csv[4] = {cs.x, cs.y, cs.z, cs.w}, wsv[4] = {ws.x, ws.y, ws.z, ws.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = exp2_hw(fminf(ct - csv[i], 0.0f));  // s > t is masked below
        v[i] = (4 * lk + i <= lr) ? g[sb][i] * e * wsv[i] : 0.0f;
      }
    }
    const i16x4 sf = __builtin_bit_cast(i16x4, u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])});
    y = mfma16k16(tr_frag4<kPS>(&sm.Xs[cur][16 * sb][0], lane), sf, y);
  }
}

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
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave: token block 16 w ..
  const int lr = lane & 15, lk = lane >> 4;                // MFMA row / k-group of this lane
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

  // ---- global reads of one chunk into registers, addressed as a uniform
  // chunk base plus 32-bit byte offsets; rows past L are clamped to the last
  // row (finite data that the zero weights of padding tokens cancel).  Issued
  // two chunks ahead of use, one chunk ahead of staging.
  u32x4 rB[RB], rC[NK];
  u32x2 rX, rZ = u32x2{0u, 0u};
  float rdt;
  const int tz = 16 * w + lr;   // token of this lane's C row, z and output
  const int tx = tid >> 2;      // token of this thread's x piece
  auto load_chunk = [&](int64_t t0) {
    const int lim = (int)(L - 1 - t0 < kQ - 1 ? L - 1 - t0 : kQ - 1);  // last row of the chunk
    const char* Bc = (const char*)(p.B + (b * L + t0) * N);
    const char* Cc = (const char*)(p.C + (b * L + t0) * N);
    const char* Xc = (const char*)(p.x + (b * L + t0) * HP + ch0);
    const char* Zc = (const char*)(p.z + (b * L + t0) * HP + ch0);
    const char* Dc = (const char*)(p.dt + (b * L + t0) * H + h);
    {  // first, so that waiting for it does not wait for the rest
      const uint32_t rd = (uint32_t)(lane < lim ? lane : lim);
      rdt = *(const float*)(Dc + rd * (uint32_t)H * 4u);
    }
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int e = tid + 256 * r;
      const int s = e / (N / 8), c8 = (e % (N / 8)) * 8;
      const uint32_t off = (uint32_t)((s < lim ? s : lim) * N + c8) * 2u;
      rB[r] = *(const u32x4*)(Bc + off);
    }
    const uint32_t rz = (uint32_t)(tz < lim ? tz : lim);
    const uint32_t offc = (rz * N + 8 * lk) * 2u;
#pragma unroll
    for (int k = 0; k < NK; ++k) rC[k] = *(const u32x4*)(Cc + offc + 64 * k);
    if constexpr (GATE) rZ = *(const u32x2*)(Zc + (rz * (uint32_t)HP + 4 * lk) * 2u);
    const uint32_t rx = (uint32_t)(tx < lim ? tx : lim);
    rX = *(const u32x2*)(Xc + (rx * (uint32_t)HP + 4 * (tid & 3)) * 2u);
  };

  // ---- step sizes, decays and weights of a chunk (wave 0, lane = token)
  auto chunk_consts = [&](ChunkConsts& kc, float raw, int nlive) {
    const float v = raw + bias;
    float dl = p.softplus ? softplus_f(v) : v;
    if (lane >= nlive) dl = 0.0f;  // padding: no decay, no input
    const float a = dl * A;
    float wt = dl;
    if constexpr (ZOH) wt = dl * zoh_phi(a, exp2_hw(a * kLog2e));
    const float c = wave_inclusive_sum(a * kLog2e);  // running sum, log2 units
    const float cb0 = lane_value(c, 15), cb1 = lane_value(c, 31), cb2 = lane_value(c, 47);
    const float cend = lane_value(c, 63);
    const float cblk = lane < 16 ? cb0 : (lane < 32 ? cb1 : (lane < 48 ? cb2 : cend));
    kc.cuml[lane] = c;
    kc.wv[lane] = wt;
    kc.fw[lane] = exp2_hw(cblk - c) * wt;
    kc.eend[lane] = exp2_hw(cend - c) * wt;
    kc.et[lane] = exp2_hw(c);
  };

  // ---- stage a chunk from the registers: B rows, the x columns (rows past
  // L as zeros), this wave's C fragment and gate, the chunk's constants
  u32x4 cC[NK];
  float gz[4] = {1.0f, 1.0f, 1.0f, 1.0f};
  auto stage = [&](int buf, int64_t t0) {
    const int nlive = (int)(L - t0 < kQ ? L - t0 : kQ);
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int e = tid + 256 * r;
      *(u32x4*)&sm.Bs[buf][e / (N / 8)][(e % (N / 8)) * 8] = rB[r];
    }
    *(u32x2*)&sm.Xs[buf][tx][4 * (tid & 3)] = tx < nlive ? rX : u32x2{0u, 0u};
#pragma unroll
    for (int k = 0; k < NK; ++k) cC[k] = rC[k];
    if constexpr (GATE) {
      gz[0] = silu_f(lo_bf(rZ.x));
      gz[1] = silu_f(hi_bf(rZ.x));
      gz[2] = silu_f(lo_bf(rZ.y));
      gz[3] = silu_f(hi_bf(rZ.y));
    }
    if (w == 0) chunk_consts(sm.cc[buf], rdt, nlive);
  };

  // Per chunk, after the barrier that publishes its staging: Y^T from the
  // state, the scores times x, the epilogue, the state update; then the next
  // chunk is staged into the other buffers and the one after it is read.
  const int64_t nchunks = (L + kQ - 1) / kQ;
  if (nchunks > 0) {
    load_chunk(0);
    stage(0, 0);
    if (nchunks > 1) load_chunk(kQ);
  }
  lds_barrier();
  for (int64_t ck = 0; ck < nchunks; ++ck) {
    const int64_t t0 = ck * kQ;
    const int nlive = (int)(L - t0 < kQ ? L - t0 : kQ);
    const int cur = (int)(ck & 1), nxt = cur ^ 1;
    const ChunkConsts& kc = sm.cc[cur];

    // ---- Y^T for token block w: D[p][t] = exp(cum_t) sum_n H[p][n] C[t][n]
    //      + sum_s x[s][p] S[t][s]; lane value i is p = 4 lk + i, t = 16 w + lr
    f32x4 y = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int k = 0; k < NK; ++k)
      y = mfma16(*(const bf16x8*)&sm.Hs[cur][lr][32 * k + 8 * lk], as_bf16x8(cC[k]), y);
    {
      const float e = kc.et[tz];
#pragma unroll
      for (int i = 0; i < 4; ++i) y[i] *= e;
    }
    switch (w) {
      case 0: scores_times_x<0, N>(sm, cur, kc, cC, lane, y); break;
      case 1: scores_times_x<1, N>(sm, cur, kc, cC, lane, y); break;
      case 2: scores_times_x<2, N>(sm, cur, kc, cC, lane, y); break;
      default: scores_times_x<3, N>(sm, cur, kc, cC, lane, y); break;
    }
    // ---- epilogue: skip, gate, store 4 channels of token tz
    if (tz < nlive) {
      const u32x2 xv = *(const u32x2*)&sm.Xs[cur][tz][4 * lk];
      const float o0 = fmaf(Dh, lo_bf(xv.x), y[0]) * gz[0];
      const float o1 = fmaf(Dh, hi_bf(xv.x), y[1]) * gz[1];
      const float o2 = fmaf(Dh, lo_bf(xv.y), y[2]) * gz[2];
      const float o3 = fmaf(Dh, hi_bf(xv.y), y[3]) * gz[3];
      char* Yc = (char*)(p.y + (b * L + t0) * HP + ch0);
      *(u32x2*)(Yc + ((uint32_t)tz * (uint32_t)HP + 4 * lk) * 2u) =
          u32x2{pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)};
    }

    // ---- state update, H^T tiles: D[n][p] = exp(cum_Q) H^T[n][p]
    //      + sum_s B[s][n] (eend_s x[s][p])
    {
      const float etot = exp2_hw(kc.cuml[kQ - 1]);
#pragma unroll
      for (int j = 0; j < NTW; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) Hacc[j][i] *= etot;
#pragma unroll
      for (int s0 = 0; s0 < kQ; s0 += 32) {
        const bf16x8 xt = tr_frag<kPS>(&sm.Xs[cur][s0][0], lane);  // x[s0 + 8 lk + j][lr]
        const float4 e0 = *(const float4*)&kc.eend[s0 + 8 * lk];
        const float4 e1 = *(const float4*)&kc.eend[s0 + 8 * lk + 4];
        const float ev[8] = {e0.x, e0.y, e0.z, e0.w, e1.x, e1.y, e1.z, e1.w};
        bf16x8 xw;
#pragma unroll
        for (int j = 0; j < 8; ++j) xw[j] = (__bf16)((float)xt[j] * ev[j]);
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
          const bf16x8 bt = tr_frag<Sm::BS>(&sm.Bs[cur][s0][16 * (w + kWaves * j)], lane);
          Hacc[j] = mfma16(bt, xw, Hacc[j]);
        }
      }
      // Hs[nxt] was last read in the previous chunk, before this chunk's barrier
#pragma unroll
      for (int j = 0; j < NTW; ++j)
        *(u32x2*)&sm.Hs[nxt][lr][16 * (w + kWaves * j) + 4 * lk] =
            u32x2{pack_bf16x2(Hacc[j][0], Hacc[j][1]), pack_bf16x2(Hacc[j][2], Hacc[j][3])};
    }

    // ---- the next chunk into the other buffers (last read in the previous
    // chunk), and the reads of the one after it
    if (ck + 1 < nchunks) {
      stage(nxt, t0 + kQ);
      if (ck + 2 < nchunks) load_chunk(t0 + 2 * kQ);
    }
    lds_barrier();
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
