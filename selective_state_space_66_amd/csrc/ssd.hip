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
// Work split: a block owns 16 of a head's P channels (one MFMA tile) for one
// batch entry and walks the chunks in order, so b * H * P / 16 blocks run at
// once (768 for 8 x 24 heads of 64: three per CU).  The block recomputes the chunk's
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
// enters LDS: each wave reads the 16 C rows of its token block in whole
// 128-byte row pieces and moves them into the operand registers with DPP row
// shifts (the same fragment serves C B^T and H C^T).
//
// Memory operations: every chunk issues the same loads and the same store
// (past the end the last chunk is read again; the output is a buffer store
// whose range ends at row L), so each wait for the loads of a chunk, issued a
// chunk ahead, counts a fixed number of later operations and waits for those
// loads only.
//
// P may be any multiple of 16; N is 64 or 128; io is bf16.
#include "ssm_device.h"
#include "ssm_launch.h"

namespace ssm66 {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) float f32x8;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(8))) short i16x8;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kQ = 64;               // tokens per chunk
constexpr int kPS = 16;              // channels per block (a head's P is a multiple of it)
constexpr int kWaves = 4;
// Word 3 of a raw buffer resource (no stride, no swizzle, 32-bit data format):
// accesses at or past the range in word 2 read 0 and write nothing.
constexpr int kBufferFlags = 0x00020000;

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

// The contractions over the states (C B^T and C H^T) take the N states in
// k-steps of 32; within a k-step, lane group lk (lanes 16 lk .. 16 lk + 15)
// holds the 8 states starting at kn(k, lk) = 64 (k / 2) + 16 lk + 8 (k % 2).
// Any split that is the same for both operands gives the same sums; this one
// lets C be read by whole 128-byte rows (see load_chunk).
__device__ __forceinline__ constexpr int kn(int k, int lk) { return 64 * (k / 2) + 16 * lk + 8 * (k % 2); }

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

// B, C and the state sit in LDS in rows of N bf16 with the 16-byte pieces of
// row r permuted: piece c is stored at c ^ swz(r).  Two access patterns meet
// in these rows: 16-byte reads of one piece by 16 lanes on rows r .. r + 15
// (the operands of the contractions over the states), and transposing reads
// in which each group of 16 lanes takes 32 bytes from each of rows r .. r + 3
// (the B operand of the state update); the staging writes whole rows.  swz
// rotates the low three bits of r by one (and folds in bit 3), which gives
// each lane of a pass its own banks in all three, with 32 banks as with 64,
// where no plain row padding serves both of the first two.
template <int N>
__device__ __forceinline__ constexpr int swz(int r) {
  return (((r << 1) & 6) | ((r >> 2) & 1)) ^ (((r >> 3) & 1) * (N == 128 ? 8 : 2));
}
// the element offset of column col within row r (col % 8 is kept)
template <int N>
__device__ __forceinline__ constexpr int sw(int r, int col) {
  return (((col >> 3) ^ swz<N>(r)) << 3) | (col & 7);
}

// tr_frag on rows stored with the permutation: the fragment of the 16 x 32
// (row x column) block at rows r0 .., columns col0 .., where rows points at
// row r0, a multiple of 16 (so swz of its rows depends on the offset only).
template <int N>
__device__ __forceinline__ bf16x8 tr_frag_sw(const __bf16* rows, int col0, int lane) {
  const int g = lane >> 4, kk = (lane & 15) >> 2, qq = lane & 3;
  const int ra = 8 * g + kk, rb = ra + 4, col = col0 + 4 * qq;
  const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(void*)(rows + ra * N + sw<N>(ra, col)));
  const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(void*)(rows + rb * N + sw<N>(rb, col)));
  const i16x8 v = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// Xs rows are 32 bytes, so the 16 lanes of a transposing read (4 rows x 4
// column quads) cover 32 banks once.  Everything a chunk reads is
// double-buffered by chunk parity, so staging the next chunk does not wait for
// the current one: one barrier per chunk.
template <int N>
struct alignas(16) SSDSmem {
  static constexpr int BS = N;
  __bf16 Bs[2][kQ][BS];         // B rows of a chunk (pieces permuted by swz)
  __bf16 Xs[2][kQ][kPS];        // this block's x columns (p contiguous)
  __bf16 Hs[2][kPS][BS];        // the state entering a chunk, bf16 (pieces permuted)
  ChunkConsts cc[2];            // per-token constants
};

struct SSDArgs {
  const bf16_bits *x, *B, *C, *z;
  const float *dt, *A, *D, *dt_bias, *h0;
  bf16_bits* y;
  float* last_state;
  int64_t batch, L, nheads, P;
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
template <int W, int N, int BS>
__device__ __forceinline__ void scores_times_x(const __bf16 (*Bs)[BS], const __bf16 (*Xs)[kPS],
                                               const ChunkConsts& kc,
                                               const u32x4 (&cC)[N / 32], int lane, f32x4& y) {
  const int lr = lane & 15, lk = lane >> 4;
  f32x4 g[W + 1];
#pragma unroll
  for (int sb = 0; sb <= W; ++sb) g[sb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int k = 0; k < N / 32; ++k)
#pragma unroll
    for (int sb = 0; sb <= W; ++sb)
      g[sb] = mfma16(*(const bf16x8*)&Bs[16 * sb + lr][sw<N>(lr, kn(k, lk))], as_bf16x8(cC[k]),
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
    y = mfma16k16(tr_frag4<kPS>(&Xs[16 * sb][0], lane), sf, y);
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
  const int64_t H = p.nheads, L = p.L, P = p.P, HP = H * P;
  const int64_t nsl = P / kPS;  // blocks per (batch entry, head)

  // XCD-aware order: consecutive block ids go round-robin to the 8 XCDs, so
  // each XCD gets a contiguous run of (batch entry, head, slice) -- the blocks
  // of one batch entry share its B and C rows in that XCD's L2.
  const int64_t nblk = (int64_t)gridDim.x, bid = blockIdx.x;
  const int64_t logical = (nblk % 8 == 0) ? (bid % 8) * (nblk / 8) + bid / 8 : bid;
  const int64_t bh = logical / nsl;
  const int64_t q = logical - bh * nsl;
  const int64_t b = bh / H, h = bh - b * H;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave: token block 16 w ..
  const int lr = lane & 15, lk = lane >> 4;                // MFMA row / k-group of this lane
  const float A = p.A[h];
  const float Dh = p.D ? p.D[h] : 0.0f;
  const float bias = p.dt_bias ? p.dt_bias[h] : 0.0f;
  const int64_t ch0 = h * P + q * kPS;      // first channel of the block in a row of x, z, y

  // ---- the state, as H^T tiles: wave w holds column tiles nt = w + 4 j;
  // lane value i is H[p = lr][n = 16 nt + 4 lk + i]
  const int64_t hrow = ((b * H + h) * P + q * kPS + lr) * N;
  f32x4 Hacc[NTW];
#pragma unroll
  for (int j = 0; j < NTW; ++j) {
    const int n = 16 * (w + kWaves * j) + 4 * lk;
    Hacc[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    if (p.h0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) Hacc[j][i] = p.h0[hrow + n + i];
    }
    *(u32x2*)&sm.Hs[0][lr][sw<N>(lr, n)] =
        u32x2{pack_bf16x2(Hacc[j][0], Hacc[j][1]), pack_bf16x2(Hacc[j][2], Hacc[j][3])};
  }

  // ---- global reads of one chunk into registers, addressed as a uniform
  // chunk base plus 32-bit byte offsets that are the same for every full
  // chunk; in a partial last chunk rows past L are clamped to the last row
  // (finite data that the zero weights of padding tokens cancel).  Issued two
  // chunks ahead of use, one chunk ahead of staging (C too: its registers
  // are copied into the operand registers when the chunk is staged).
  u32x4 rB[RB], rC[NK];
  u32x2 rX, rZ = u32x2{0u, 0u};
  float rdt;
  const int tz = 16 * w + lr;   // token of this lane's C row, z and output
  const int tx = tid >> 2;      // token of this thread's x piece
  const int sB = tid / (N / 8), cB8 = (tid % (N / 8)) * 8;  // first B piece: row, column
  constexpr int kRowsPerPiece = 256 / (N / 8);                // B rows between pieces
  const uint32_t offB = (uint32_t)(sB * N + cB8) * 2u;
  // C: wave w reads the 16 rows of its token block as whole 128-byte pieces
  // of rows: load j covers rows 16 w + 8 (j % 2) .. + 7, bytes 128 (j / 2) ..
  // + 127 of each; lane (lk, m) takes row + m % 8, 16 bytes at 16 (2 lk + m / 8).
  const int crow = 16 * w + (lr & 7), cpiece = 2 * lk + (lr >> 3);
  const uint32_t offC = (uint32_t)(crow * N + 8 * cpiece) * 2u;
  const uint32_t offZ = ((uint32_t)tz * (uint32_t)HP + 4 * lk) * 2u;
  const uint32_t offX = ((uint32_t)tx * (uint32_t)HP + 4 * (tid & 3)) * 2u;
  // dt is used by wave 0 only (one token per lane, 64 cache lines); the
  // other waves issue the same load on one address, so that every wave keeps
  // the same count of memory operations in flight
  const uint32_t offD = w == 0 ? (uint32_t)lane * (uint32_t)H * 4u : 0u;
  auto load_chunk = [&](int64_t t0) {
    const char* Bc = (const char*)(p.B + (b * L + t0) * N);
    const char* Cc = (const char*)(p.C + (b * L + t0) * N);
    const char* Xc = (const char*)(p.x + (b * L + t0) * HP + ch0);
    const char* Zc = (const char*)(p.z + (b * L + t0) * HP + ch0);
    const char* Dc = (const char*)(p.dt + (b * L + t0) * H + h);
    if (t0 + kQ <= L) {
      rdt = *(const float*)(Dc + offD);  // first, so that waiting for it does not wait for the rest
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        const char* Bcr = Bc + r * kRowsPerPiece * N * 2;  // uniform: the offset stays 32-bit
        rB[r] = *(const u32x4*)(Bcr + offB);
      }
#pragma unroll
      for (int j = 0; j < NK; ++j)
        rC[j] = *(const u32x4*)(Cc + (offC + (uint32_t)((8 * (j % 2) * N + 64 * (j / 2)) * 2)));
      if constexpr (GATE) rZ = *(const u32x2*)(Zc + offZ);
      rX = *(const u32x2*)(Xc + offX);
    } else {
      const int lim = (int)(L - 1 - t0);  // last row of the chunk, < kQ - 1
      rdt = *(const float*)(Dc + (w == 0 ? (uint32_t)(lane < lim ? lane : lim) * (uint32_t)H * 4u : 0u));
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        const int sr = sB + r * kRowsPerPiece;
        rB[r] = *(const u32x4*)(Bc + (uint32_t)((sr < lim ? sr : lim) * N + cB8) * 2u);
      }
      const uint32_t rz = (uint32_t)(tz < lim ? tz : lim);
#pragma unroll
      for (int j = 0; j < NK; ++j) {
        const int cr = crow + 8 * (j % 2);
        rC[j] = *(const u32x4*)(Cc + (uint32_t)((cr < lim ? cr : lim) * N + 8 * cpiece + 64 * (j / 2)) * 2u);
      }
      if constexpr (GATE) rZ = *(const u32x2*)(Zc + (rz * (uint32_t)HP + 4 * lk) * 2u);
      const uint32_t rx = (uint32_t)(tx < lim ? tx : lim);
      rX = *(const u32x2*)(Xc + (rx * (uint32_t)HP + 4 * (tid & 3)) * 2u);
    }
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
      const int row = sB + r * kRowsPerPiece;
      *(u32x4*)&sm.Bs[buf][row][sw<N>(row, cB8)] = rB[r];
    }
    *(u32x2*)&sm.Xs[buf][tx][4 * (tid & 3)] = tx < nlive ? rX : u32x2{0u, 0u};
    // C into the operand layout (lane group lk, lane m = token 16 w + m,
    // states kn(k, lk) ..): within each 16-lane row, the 8 lanes m >= 8 of the
    // rows-0..7 load and the 8 lanes m < 8 of the rows-8..15 load trade places
    // (DPP row shifts by 8 that write only half of each row).  The halves kept
    // are first copied into new registers: were the shifts written over the
    // loaded registers, the next chunk's loads would need other registers and
    // the loop would end by moving them back, waiting there for those loads.
#pragma unroll
    for (int h = 0; h < NK / 2; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r0 = (int)rC[2 * h][i], r1 = (int)rC[2 * h + 1][i];
        int k0, k1;
        asm("v_mov_b32 %0, %1" : "=v"(k0) : "v"(r0));
        asm("v_mov_b32 %0, %1" : "=v"(k1) : "v"(r1));
        cC[2 * h][i] = (uint32_t)__builtin_amdgcn_update_dpp(k0, r1, 0x118, 0xf, 0xc, false);
        cC[2 * h + 1][i] = (uint32_t)__builtin_amdgcn_update_dpp(k1, r0, 0x108, 0xf, 0x3, false);
      }
    if constexpr (GATE) {
      gz[0] = silu_f(lo_bf(rZ.x));
      gz[1] = silu_f(hi_bf(rZ.x));
      gz[2] = silu_f(lo_bf(rZ.y));
      gz[3] = silu_f(hi_bf(rZ.y));
    }
    if (w == 0) chunk_consts(sm.cc[buf], rdt, nlive);
  };

  const int64_t nchunks = (L + kQ - 1) / kQ;
  const int64_t tlast = (nchunks - 1) * kQ;  // first token of the last chunk
  if (nchunks > 0) {
    load_chunk(0);
    stage(0, 0);
    load_chunk(nchunks > 1 ? kQ : 0);
    // a store that writes nothing (empty range), so that the loop is entered
    // with the same memory operations in flight as each chunk leaves it
    const __amdgpu_buffer_rsrc_t none =
        __builtin_amdgcn_make_buffer_rsrc((void*)p.y, (short)0, 0, kBufferFlags);
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{0u, 0u}, none, (int)offZ, 0, 0);
  }
  lds_barrier();

  // One chunk, after the barrier that publishes its staging: Y^T from the
  // state, the scores times x, the epilogue, the state update; then the next
  // chunk is staged into the other buffers, the one after it is read, and the
  // chunk's output is stored.
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
      y = mfma16(*(const bf16x8*)&sm.Hs[cur][lr][sw<N>(lr, kn(k, lk))], as_bf16x8(cC[k]), y);
    {
      const float e = kc.et[tz];
#pragma unroll
      for (int i = 0; i < 4; ++i) y[i] *= e;
    }
    switch (w) {
      case 0: scores_times_x<0, N, Sm::BS>(sm.Bs[cur], sm.Xs[cur], kc, cC, lane, y); break;
      case 1: scores_times_x<1, N, Sm::BS>(sm.Bs[cur], sm.Xs[cur], kc, cC, lane, y); break;
      case 2: scores_times_x<2, N, Sm::BS>(sm.Bs[cur], sm.Xs[cur], kc, cC, lane, y); break;
      default: scores_times_x<3, N, Sm::BS>(sm.Bs[cur], sm.Xs[cur], kc, cC, lane, y); break;
    }
    // ---- epilogue: skip, gate; 4 channels of token tz, stored at the end
    // of the chunk
    u32x2 yout;
    {
      const u32x2 xv = *(const u32x2*)&sm.Xs[cur][tz][4 * lk];
      const float o0 = fmaf(Dh, lo_bf(xv.x), y[0]) * gz[0];
      const float o1 = fmaf(Dh, hi_bf(xv.x), y[1]) * gz[1];
      const float o2 = fmaf(Dh, lo_bf(xv.y), y[2]) * gz[2];
      const float o3 = fmaf(Dh, hi_bf(xv.y), y[3]) * gz[3];
      yout = u32x2{pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)};
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
        const f32x8 ev = *(const f32x8*)&kc.eend[s0 + 8 * lk];
        const bf16x8 xw = __builtin_convertvector(__builtin_convertvector(xt, f32x8) * ev, bf16x8);
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
          const bf16x8 bt = tr_frag_sw<N>(&sm.Bs[cur][s0][0], 16 * (w + kWaves * j), lane);
          Hacc[j] = mfma16(bt, xw, Hacc[j]);
        }
      }
      // Hs[nxt] was last read in the previous chunk, before this chunk's barrier
#pragma unroll
      for (int j = 0; j < NTW; ++j)
        *(u32x2*)&sm.Hs[nxt][lr][sw<N>(lr, 16 * (w + kWaves * j) + 4 * lk)] =
            u32x2{pack_bf16x2(Hacc[j][0], Hacc[j][1]), pack_bf16x2(Hacc[j][2], Hacc[j][3])};
    }

    // ---- the next chunk into the other buffers (last read in the previous
    // chunk), the reads of the one after it, then this chunk's output.  All of
    // it is issued on every chunk, so that each wait for a load counts a fixed
    // number of later memory operations: past the end the staged buffers are
    // never read and the last chunk is read again; the store is a buffer store
    // whose range ends at row L, so the hardware drops the rows past it.
    stage(nxt, t0 + kQ);
    load_chunk(t0 + 2 * kQ < L ? t0 + 2 * kQ : tlast);
    {
      const __amdgpu_buffer_rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(p.y + (b * L + t0) * HP + ch0), (short)0, nlive * (int)HP * 2, kBufferFlags);
      __builtin_amdgcn_raw_buffer_store_b64(yout, yr, (int)offZ, 0, 0);
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

// ---- the grouped form, for shapes with enough slices to give every CU a
// block: a block of kGroups x 4 waves takes kGroups slices (16 channels each)
// of one batch entry.  The chunk's B and C rows -- the same for every head --
// are read from memory once per block into LDS and shared by the groups,
// which cuts the block's reads of them kGroups-fold; each group keeps its own
// x columns, state, constants and output, exactly as the one-slice kernel
// above (the same products, in the same order, so the same results).  Where a
// batch entry's slices do not fill its last block, the spare groups compute
// on the last slice and store nothing.
constexpr int kGroups = 3;

template <int N>
struct alignas(16) SSDGroupSmem {
  static constexpr int BS = N;
  __bf16 Bs[2][kQ][BS];                  // B rows of a chunk (shared; pieces permuted by swz)
  __bf16 Cs[2][kQ][BS];                  // C rows of a chunk (shared; pieces permuted)
  __bf16 Xs[kGroups][2][kQ][kPS];        // each group's x columns
  __bf16 Hs[kGroups][2][kPS][BS];        // each group's state, bf16 (pieces permuted)
  ChunkConsts cc[kGroups][2];            // each group's per-token constants
};

template <int N, bool ZOH, bool GATE>
__global__ __launch_bounds__(64 * kWaves * kGroups, 1) void ssd_fwd_grouped_kernel(
    const SSDArgs p) {
  using Sm = SSDGroupSmem<N>;
  __shared__ Sm sm;
  constexpr int NK = N / 32;
  constexpr int NTW = N / 16 / kWaves;
  constexpr int NT = 64 * kWaves * kGroups;   // threads
  constexpr int PIECES = kQ * N / 8;          // 16-byte pieces of B (and of C) per chunk
  constexpr int RBC = (2 * PIECES + NT - 1) / NT;
  static_assert(NTW >= 1, "N is 64 or 128");
  const int64_t H = p.nheads, L = p.L, P = p.P, HP = H * P;
  const int64_t nsl = P / kPS;                         // slices per head
  const int64_t SB = H * nsl;                          // slices per batch entry
  const int64_t nbb = (SB + kGroups - 1) / kGroups;    // blocks per batch entry

  // XCD-aware order, as the one-slice kernel: an XCD's blocks are consecutive
  // logical blocks, i.e. mostly one batch entry, whose B and C stay in its L2
  const int64_t nblk = (int64_t)gridDim.x, bid = blockIdx.x;
  const int64_t logical = (nblk % 8 == 0) ? (bid % 8) * (nblk / 8) + bid / 8 : bid;
  const int64_t b = logical / nbb, slot = logical - b * nbb;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = wv / kWaves, w = wv % kWaves;          // group; token block 16 w ..
  const int tg = tid - g * 64 * kWaves;                // thread within the group
  const int lr = lane & 15, lk = lane >> 4;
  const int64_t sl0 = slot * kGroups + g;
  const bool live_group = sl0 < SB;
  const int64_t slc = live_group ? sl0 : SB - 1;
  const int64_t h = slc / nsl, q = slc - h * nsl;
  const float A = p.A[h];
  const float Dh = p.D ? p.D[h] : 0.0f;
  const float bias = p.dt_bias ? p.dt_bias[h] : 0.0f;
  const int64_t ch0 = h * P + q * kPS;

  const int64_t hrow = ((b * H + h) * P + q * kPS + lr) * N;
  f32x4 Hacc[NTW];
#pragma unroll
  for (int j = 0; j < NTW; ++j) {
    const int n = 16 * (w + kWaves * j) + 4 * lk;
    Hacc[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    if (p.h0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) Hacc[j][i] = p.h0[hrow + n + i];
    }
    *(u32x2*)&sm.Hs[g][0][lr][sw<N>(lr, n)] =
        u32x2{pack_bf16x2(Hacc[j][0], Hacc[j][1]), pack_bf16x2(Hacc[j][2], Hacc[j][3])};
  }

  // ---- global reads of one chunk, issued two chunks ahead of use: the block
  // reads B and C (piece e = tid + NT r: B for e < PIECES, then C; pieces
  // past the end load the last one again and are not staged), each group its
  // x columns, each wave the gate of its tokens, wave 0 of a group its step
  // sizes (the group's other waves load one address, as in the one-slice
  // kernel).  Rows past L are clamped to the last row.
  u32x4 rBC[RBC];
  u32x2 rX, rZ = u32x2{0u, 0u};
  float rdt;
  const int tz = 16 * w + lr;
  const int tx = tg >> 2;
  const uint32_t offZ = ((uint32_t)tz * (uint32_t)HP + 4 * lk) * 2u;
  const uint32_t offX = ((uint32_t)tx * (uint32_t)HP + 4 * (tg & 3)) * 2u;
  const uint32_t offD = w == 0 ? (uint32_t)lane * (uint32_t)H * 4u : 0u;
  auto piece = [&](int r, int& row, int& col, bool& isC, bool& staged) {
    const int e0 = tid + NT * r;
    staged = e0 < 2 * PIECES;
    const int e = staged ? e0 : 2 * PIECES - 1;
    isC = e >= PIECES;
    const int ep = isC ? e - PIECES : e;
    row = ep / (N / 8);
    col = (ep % (N / 8)) * 8;
  };
  auto load_chunk = [&](int64_t t0) {
    const int lim = (int)(L - 1 - t0 < kQ - 1 ? L - 1 - t0 : kQ - 1);  // last row of the chunk
    const char* Bc = (const char*)(p.B + (b * L + t0) * N);
    const char* Cc = (const char*)(p.C + (b * L + t0) * N);
    const char* Xc = (const char*)(p.x + (b * L + t0) * HP + ch0);
    const char* Zc = (const char*)(p.z + (b * L + t0) * HP + ch0);
    const char* Dc = (const char*)(p.dt + (b * L + t0) * H + h);
    const int ld = lane < lim ? lane : lim;
    rdt = *(const float*)(Dc + (w == 0 ? (uint32_t)ld * (uint32_t)H * 4u : 0u));
#pragma unroll
    for (int r = 0; r < RBC; ++r) {
      int row, col;
      bool isC, staged;
      piece(r, row, col, isC, staged);
      const uint32_t off = (uint32_t)((row < lim ? row : lim) * N + col) * 2u;
      rBC[r] = *(const u32x4*)((isC ? Cc : Bc) + off);
    }
    const uint32_t rz = (uint32_t)(tz < lim ? tz : lim);
    if constexpr (GATE) rZ = *(const u32x2*)(Zc + (rz * (uint32_t)HP + 4 * lk) * 2u);
    const uint32_t rx = (uint32_t)(tx < lim ? tx : lim);
    rX = *(const u32x2*)(Xc + (rx * (uint32_t)HP + 4 * (tg & 3)) * 2u);
    (void)offD;
  };

  auto chunk_consts = [&](ChunkConsts& kc, float raw, int nlive) {
    const float v = raw + bias;
    float dl = p.softplus ? softplus_f(v) : v;
    if (lane >= nlive) dl = 0.0f;
    const float a = dl * A;
    float wt = dl;
    if constexpr (ZOH) wt = dl * zoh_phi(a, exp2_hw(a * kLog2e));
    const float c = wave_inclusive_sum(a * kLog2e);
    const float cb0 = lane_value(c, 15), cb1 = lane_value(c, 31), cb2 = lane_value(c, 47);
    const float cend = lane_value(c, 63);
    const float cblk = lane < 16 ? cb0 : (lane < 32 ? cb1 : (lane < 48 ? cb2 : cend));
    kc.cuml[lane] = c;
    kc.wv[lane] = wt;
    kc.fw[lane] = exp2_hw(cblk - c) * wt;
    kc.eend[lane] = exp2_hw(cend - c) * wt;
    kc.et[lane] = exp2_hw(c);
  };

  float gz[4] = {1.0f, 1.0f, 1.0f, 1.0f};
  auto stage = [&](int buf, int64_t t0) {
    const int nlive = (int)(L - t0 < kQ ? L - t0 : kQ);
#pragma unroll
    for (int r = 0; r < RBC; ++r) {
      int row, col;
      bool isC, staged;
      piece(r, row, col, isC, staged);
      if (staged) *(u32x4*)(isC ? &sm.Cs[buf][row][sw<N>(row, col)] : &sm.Bs[buf][row][sw<N>(row, col)]) = rBC[r];
    }
    *(u32x2*)&sm.Xs[g][buf][tx][4 * (tg & 3)] = tx < nlive ? rX : u32x2{0u, 0u};
    if constexpr (GATE) {
      gz[0] = silu_f(lo_bf(rZ.x));
      gz[1] = silu_f(hi_bf(rZ.x));
      gz[2] = silu_f(lo_bf(rZ.y));
      gz[3] = silu_f(hi_bf(rZ.y));
    }
    if (w == 0) chunk_consts(sm.cc[g][buf], rdt, nlive);
  };

  const int64_t nchunks = (L + kQ - 1) / kQ;
  const int64_t tlast = (nchunks - 1) * kQ;
  if (nchunks > 0) {
    load_chunk(0);
    stage(0, 0);
    load_chunk(nchunks > 1 ? kQ : 0);
    // a store that writes nothing, so that every chunk starts with the same
    // memory operations in flight (as in the one-slice kernel)
    const __amdgpu_buffer_rsrc_t none =
        __builtin_amdgcn_make_buffer_rsrc((void*)p.y, (short)0, 0, kBufferFlags);
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{0u, 0u}, none, (int)offZ, 0, 0);
  }
  lds_barrier();

  for (int64_t ck = 0; ck < nchunks; ++ck) {
    const int64_t t0 = ck * kQ;
    const int nlive = (int)(L - t0 < kQ ? L - t0 : kQ);
    const int cur = (int)(ck & 1), nxt = cur ^ 1;
    const ChunkConsts& kc = sm.cc[g][cur];

    u32x4 cC[NK];
#pragma unroll
    for (int k = 0; k < NK; ++k) cC[k] = *(const u32x4*)&sm.Cs[cur][tz][sw<N>(tz, kn(k, lk))];

    f32x4 y = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int k = 0; k < NK; ++k)
      y = mfma16(*(const bf16x8*)&sm.Hs[g][cur][lr][sw<N>(lr, kn(k, lk))], as_bf16x8(cC[k]), y);
    {
      const float e = kc.et[tz];
#pragma unroll
      for (int i = 0; i < 4; ++i) y[i] *= e;
    }
    switch (w) {
      case 0: scores_times_x<0, N, Sm::BS>(sm.Bs[cur], sm.Xs[g][cur], kc, cC, lane, y); break;
      case 1: scores_times_x<1, N, Sm::BS>(sm.Bs[cur], sm.Xs[g][cur], kc, cC, lane, y); break;
      case 2: scores_times_x<2, N, Sm::BS>(sm.Bs[cur], sm.Xs[g][cur], kc, cC, lane, y); break;
      default: scores_times_x<3, N, Sm::BS>(sm.Bs[cur], sm.Xs[g][cur], kc, cC, lane, y); break;
    }
    u32x2 yout;
    {
      const u32x2 xv = *(const u32x2*)&sm.Xs[g][cur][tz][4 * lk];
      const float o0 = fmaf(Dh, lo_bf(xv.x), y[0]) * gz[0];
      const float o1 = fmaf(Dh, hi_bf(xv.x), y[1]) * gz[1];
      const float o2 = fmaf(Dh, lo_bf(xv.y), y[2]) * gz[2];
      const float o3 = fmaf(Dh, hi_bf(xv.y), y[3]) * gz[3];
      yout = u32x2{pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)};
    }
    {
      const float etot = exp2_hw(kc.cuml[kQ - 1]);
#pragma unroll
      for (int j = 0; j < NTW; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) Hacc[j][i] *= etot;
#pragma unroll
      for (int s0 = 0; s0 < kQ; s0 += 32) {
        const bf16x8 xt = tr_frag<kPS>(&sm.Xs[g][cur][s0][0], lane);
        const f32x8 ev = *(const f32x8*)&kc.eend[s0 + 8 * lk];
        const bf16x8 xw = __builtin_convertvector(__builtin_convertvector(xt, f32x8) * ev, bf16x8);
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
          const bf16x8 bt = tr_frag_sw<N>(&sm.Bs[cur][s0][0], 16 * (w + kWaves * j), lane);
          Hacc[j] = mfma16(bt, xw, Hacc[j]);
        }
      }
#pragma unroll
      for (int j = 0; j < NTW; ++j)
        *(u32x2*)&sm.Hs[g][nxt][lr][sw<N>(lr, 16 * (w + kWaves * j) + 4 * lk)] =
            u32x2{pack_bf16x2(Hacc[j][0], Hacc[j][1]), pack_bf16x2(Hacc[j][2], Hacc[j][3])};
    }
    stage(nxt, t0 + kQ);
    load_chunk(t0 + 2 * kQ < L ? t0 + 2 * kQ : tlast);
    {
      // a spare group's range is empty: its rows are not stored
      const int rows = live_group ? nlive : 0;
      const __amdgpu_buffer_rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(p.y + (b * L + t0) * HP + ch0), (short)0, rows * (int)HP * 2, kBufferFlags);
      __builtin_amdgcn_raw_buffer_store_b64(yout, yr, (int)offZ, 0, 0);
    }
    lds_barrier();
  }

  if (p.last_state && live_group) {
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
      const int n = 16 * (w + kWaves * j) + 4 * lk;
#pragma unroll
      for (int i = 0; i < 4; ++i) p.last_state[hrow + n + i] = Hacc[j][i];
    }
  }
}

// The grouped kernel where it gives every CU at least one block (256 CUs),
// else the one-slice kernel (three blocks per CU, more blocks in flight).
constexpr int64_t kGroupedMinBlocks = 256;

template <int N, bool ZOH, bool GATE>
hipError_t ssd_launch(const SSDArgs& a, hipStream_t stream) {
  const int64_t slices = a.nheads * (a.P / kPS);
  const int64_t grouped = a.batch * ((slices + kGroups - 1) / kGroups);
  if (grouped >= kGroupedMinBlocks) {
    if (grouped > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((ssd_fwd_grouped_kernel<N, ZOH, GATE>), dim3((unsigned)grouped),
                       dim3(64 * kWaves * kGroups), 0, stream, a);
    return hipGetLastError();
  }
  const int64_t nblk = a.batch * slices;
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
  a.batch = q.batch; a.L = q.L; a.nheads = q.nheads; a.P = q.P; a.softplus = q.softplus;
  if (q.P < kPS || q.P % kPS != 0) return hipErrorInvalidValue;
  if (q.N == 128) return ssd_modes<128>(a, zoh, gate, stream);
  if (q.N == 64) return ssd_modes<64>(a, zoh, gate, stream);
  return hipErrorInvalidValue;
}

}  // namespace ssm66
