// scan_tpar.hip -- the selective scan with time across lanes: the recurrence
// composed as an associative scan of affine maps (gfx950).
//
// "Mamba and selective state spaces" (zerotofrontier.app/ssm/mamba), "Selection
// breaks the convolution": with input-dependent abar_t and bbar_t the state
// update h_t = abar_t h_{t-1} + bbar_t u_t is still a first-order linear
// recurrence, and composing two of its steps is associative:
//   (a1, b1) then (a2, b2)  =  (a2 a1, a2 b1 + b2),
// so a prefix over T tokens takes O(log T) combine steps ("State-space models
// & Mamba", "3.3 Efficient implementation: the hardware-aware scan").
//
// Three levels.  A block owns one (batch entry, channel) and walks the
// sequence in chunks of 256 tokens; its 4 waves take 64 tokens each, one per
// lane.  (1) Lanes: for each state n the lane forms its token's pair
// (abar, bbar u) and the wave scans the 64 pairs with DPP (row shifts by 1, 2,
// 4, 8, then the row-15 and row-31 broadcasts).  (2) Waves: each wave's total
// pair goes to LDS; after one barrier lane n of every wave composes the carry
// entering the chunk with the totals of the waves before it.  (3) Chunks: the
// composition over all four waves is the carry into the next chunk.  Each
// lane then has h_t = A_t carry + B_t for every state and forms
// y_t = sum_n C_t[n] h_t[n] + D u_t, gated by silu(z_t).
//
// The per-state form follows the sequential kernel: exponential-Euler
// bbar = Delta B; ZOH keeps g = A h, whose step g_t = abar g + (abar - 1) u B
// has bbar u = fma(abar, uB, -uB) (one rounding), when |A| >= 1/2, else
// bbar = Delta B phi(Delta A).  A document start (reset) zeroes the state
// before its token: its pair is (0, bbar u).  Padding past a sequence's length
// is the identity pair (1, 0) and outputs 0.
//
// The pairs cost about twice the sequential update, so this kernel is chosen
// only where (batch x channels x states) is too small to fill the GPU with
// sequential lanes: long sequences of few, narrow rows.
#include <type_traits>

#include "ssm_device.h"
#include "ssm_launch.h"
#include "ssm_wave8.h"

namespace ssm66 {

namespace {

constexpr int kTW = 4;        // waves per block
constexpr int kTT = 64 * kTW; // tokens per chunk
constexpr int kNMax = 16;     // largest state size

// The inclusive pair scan over the 64 lanes for four states at once: lane i
// ends with the composition of the pairs of lanes 0..i (row shifts by 1, 2, 4,
// 8, then the last lane of rows 0 and 2 into rows 1 and 3, and lane 31 into
// rows 2 and 3).  One combine step applies the pair of the lane the DPP
// control addresses (earlier tokens) first,
//   b <- a * b_src + b,  a <- a * a_src,
// as v_fmac_f32 and v_mul_f32 with a DPP source operand.  With bound_ctrl
// off, a lane with no source lane (or in a row outside the row mask) is not
// written, i.e. it keeps its pair: the identity (1, 0) is never materialised.
// A VALU write followed by a DPP read of the same VGPR needs two wait states:
// the four states' instructions are interleaved so that three others separate
// each write from the DPP read of its result, and only the block's first
// read (of values the compiler has just written) waits.
#define SSM66_STEP4(CTRL)                                         \
  "v_fmac_f32_dpp %0, %0, %4 " CTRL " bank_mask:0xf\n\t"        \
  "v_fmac_f32_dpp %1, %1, %5 " CTRL " bank_mask:0xf\n\t"        \
  "v_fmac_f32_dpp %2, %2, %6 " CTRL " bank_mask:0xf\n\t"        \
  "v_fmac_f32_dpp %3, %3, %7 " CTRL " bank_mask:0xf\n\t"        \
  "v_mul_f32_dpp %4, %4, %4 " CTRL " bank_mask:0xf\n\t"         \
  "v_mul_f32_dpp %5, %5, %5 " CTRL " bank_mask:0xf\n\t"         \
  "v_mul_f32_dpp %6, %6, %6 " CTRL " bank_mask:0xf\n\t"         \
  "v_mul_f32_dpp %7, %7, %7 " CTRL " bank_mask:0xf\n\t"

__device__ __forceinline__ void pair_scan4(float (&a)[4], float (&b)[4]) {
  asm volatile("s_nop 1\n\t"
               SSM66_STEP4("row_shr:1 row_mask:0xf")
               SSM66_STEP4("row_shr:2 row_mask:0xf")
               SSM66_STEP4("row_shr:4 row_mask:0xf")
               SSM66_STEP4("row_shr:8 row_mask:0xf")
               SSM66_STEP4("row_bcast:15 row_mask:0xa")
               SSM66_STEP4("row_bcast:31 row_mask:0xc")
               : "+v"(b[0]), "+v"(b[1]), "+v"(b[2]), "+v"(b[3]),
                 "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]));
}

// The same scan where only b is wanted afterwards: the last level updates b
// alone (a is left at the previous level's values).  The trailing s_nop
// gives a DPP read of b right after the block its two wait states.
__device__ __forceinline__ void pair_scan4_b(float (&a)[4], float (&b)[4]) {
  asm volatile("s_nop 1\n\t"
               SSM66_STEP4("row_shr:1 row_mask:0xf")
               SSM66_STEP4("row_shr:2 row_mask:0xf")
               SSM66_STEP4("row_shr:4 row_mask:0xf")
               SSM66_STEP4("row_shr:8 row_mask:0xf")
               SSM66_STEP4("row_bcast:15 row_mask:0xa")
               "v_fmac_f32_dpp %0, %0, %4 row_bcast:31 row_mask:0xc bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %1, %1, %5 row_bcast:31 row_mask:0xc bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %2, %2, %6 row_bcast:31 row_mask:0xc bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %3, %3, %7 row_bcast:31 row_mask:0xc bank_mask:0xf\n\t"
               "s_nop 1"
               : "+v"(b[0]), "+v"(b[1]), "+v"(b[2]), "+v"(b[3]),
                 "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]));
}
#undef SSM66_STEP4

__device__ __forceinline__ float lane_bcast(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// Pointers are separate __restrict__ arguments; y must not overlap any input,
// and last_state none but h0 (read before the first chunk, written after the
// last).
// NF: N == 16 with 16-byte-aligned B and C, whose rows are read as 16-byte
// vectors.  CKPT: also write the state before every 16th token to ckpt
// (batch, ceil(L / 16), dim, N).
template <typename IO, bool ZOH, bool GATE, bool NF, bool CKPT>
__global__ __launch_bounds__(64 * kTW) void scan_tpar_kernel(
    const IO* __restrict__ u, const IO* __restrict__ dr, const float* __restrict__ Am,
    const IO* __restrict__ Bm, const IO* __restrict__ Cm, const float* __restrict__ Dm,
    const IO* __restrict__ zz, const float* __restrict__ bias_v, const float* h0,
    const int32_t* __restrict__ seq_lens, const uint8_t* __restrict__ reset,
    IO* __restrict__ y, float* last_state, float* __restrict__ ckpt, const int64_t L,
    const int64_t dim, const int N, const int softplus) {
  __shared__ float2 tot[2][kTW][kNMax];  // per chunk parity, wave, state: the wave's total pair
  __shared__ float cst[2][kNMax];        // per state: A log2(e); readout factor (1/A for the g form)

  // XCD-aware order: each XCD gets a contiguous run of channels, which share
  // the 128-byte lines of u, Delta, z and y in its L2.
  const int64_t nblk = (int64_t)gridDim.x, bid = blockIdx.x;
  const int64_t logical = (nblk % 8 == 0) ? (bid % 8) * (nblk / 8) + bid / 8 : bid;
  const int64_t b = logical / dim, c = logical - b * dim;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // per-state constants: lane n holds state n's; the loop reads them from LDS
  // (uniform values in vector registers, not one scalar register each)
  const float a_l = lane < N ? Am[c * N + lane] : 0.0f;
  const bool fast_l = ZOH && fabsf(a_l) >= 0.5f;  // ZOH g form for this state
  const float ca_l = fast_l ? 1.0f / a_l : 0.0f;
  const uint64_t fast_mask = __ballot(fast_l);
  const bool all_fast = ZOH && (~fast_mask & ((1ull << N) - 1)) == 0;  // uniform
  if (w == 0 && lane < kNMax) {
    cst[0][lane] = a_l * kLog2e;
    cst[1][lane] = fast_l ? ca_l : (ZOH ? 1.0f : 0.0f);  // readout weight of the carried value
  }
  lds_barrier();  // cst is read by every wave from the first chunk on
  const float bias = bias_v ? bias_v[c] : 0.0f;
  const float dskip = Dm ? Dm[c] : 0.0f;
  // the carry into the chunk, state n = lane (lanes < N), in g units where fast
  float carry = 0.0f;
  const int64_t nck = (L + 15) / 16;  // checkpoints per sequence (CKPT)
  if (lane < N) {
    const float hv = h0 ? h0[(b * dim + c) * N + lane] : 0.0f;
    carry = fast_l ? a_l * hv : hv;
    if (CKPT && w == 0 && L > 0) ckpt[(b * nck * dim + c) * N + lane] = hv;
  }
  int64_t Leff = L;
  if (seq_lens) {
    const int64_t sl = seq_lens[b];
    Leff = sl < 0 ? 0 : (sl < L ? sl : L);
  }

  // raw inputs of this lane's token, read a chunk ahead: a uniform chunk base
  // plus a 32-bit lane offset, clamped to the last token (no branch around a
  // load); the host guarantees kTT * dim < 2^31
  const int tl0 = 64 * w + lane;  // this lane's token within a chunk
  float ru = 0.0f, rd = 0.0f, rz = 0.0f;
  float rB[kNMax], rC[kNMax];
  uint8_t rr = 0;
  auto load = [&](int64_t t0) {
    const int64_t lim = L - 1 - t0;
    const uint32_t tl = (uint32_t)(tl0 < lim ? tl0 : lim);
    const int64_t row0 = b * L + t0;
    const uint32_t xo = tl * (uint32_t)dim;
    ru = to_f32(u[row0 * dim + c + xo]);
    rd = to_f32(dr[row0 * dim + c + xo]);
    if constexpr (GATE) rz = to_f32(zz[row0 * dim + c + xo]);
    const IO* Bb = Bm + row0 * N;
    const IO* Cb = Cm + row0 * N;
    if constexpr (NF) {
      if constexpr (sizeof(IO) == 2) {
        typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const u32x4 vb = *(const u32x4*)(Bb + tl * 16u + 8 * q);
          const u32x4 vc = *(const u32x4*)(Cb + tl * 16u + 8 * q);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            rB[8 * q + 2 * j] = __uint_as_float(vb[j] << 16);
            rB[8 * q + 2 * j + 1] = __uint_as_float(vb[j] & 0xffff0000u);
            rC[8 * q + 2 * j] = __uint_as_float(vc[j] << 16);
            rC[8 * q + 2 * j + 1] = __uint_as_float(vc[j] & 0xffff0000u);
          }
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 vb = *(const float4*)(Bb + tl * 16u + 4 * q);
          const float4 vc = *(const float4*)(Cb + tl * 16u + 4 * q);
          rB[4 * q] = vb.x; rB[4 * q + 1] = vb.y; rB[4 * q + 2] = vb.z; rB[4 * q + 3] = vb.w;
          rC[4 * q] = vc.x; rC[4 * q + 1] = vc.y; rC[4 * q + 2] = vc.z; rC[4 * q + 3] = vc.w;
        }
      }
    } else {
#pragma unroll
      for (int n = 0; n < kNMax; ++n) {
        const uint32_t e = tl * (uint32_t)N + (uint32_t)(n < N ? n : N - 1);
        rB[n] = to_f32(Bb[e]);
        rC[n] = to_f32(Cb[e]);
      }
    }
    if (reset) rr = reset[row0 + tl];
  };

  const int64_t nchunks = (L + kTT - 1) / kTT;
  if (nchunks > 0) load(0);
  for (int64_t ck = 0; ck < nchunks; ++ck) {
    const int64_t t0 = ck * kTT;
    const int64_t t = t0 + 64 * w + lane;
    const bool live = t < Leff;
    const float x = live ? ru : 0.0f;
    const float v = rd + bias;
    const float dl = live ? (softplus ? softplus_f(v) : v) : 0.0f;
    const float gz = GATE ? silu_f(rz) : 1.0f;
    const bool rst = live && rr != 0;
    // padding tokens take B = 0 (whatever their inputs hold), so that their
    // pair is exactly the identity (1, 0)
    float Bv[kNMax], Cv[kNMax];
#pragma unroll
    for (int n = 0; n < kNMax; ++n) {
      Bv[n] = live ? rB[n] : 0.0f;
      Cv[n] = rC[n];
    }
    if (ck + 1 < nchunks) load(t0 + kTT);

    // (1) per state: the token's pair, scanned over the wave's 64 tokens.  The
    // per-state form is chosen once per block when every state takes the
    // same one (FORM 0: Euler, 1: ZOH g form, 2: ZOH, per state).
    float pa[kNMax], pb[kNMax];
    // the states are formed and scanned four at a time; with a state size
    // below 16 the states of the last group past N are finite dummies (A = 0)
    // that are never read out, and groups wholly past N are skipped
    auto pairs = [&](auto form_tag) {
      constexpr int FORM = decltype(form_tag)::value;
#pragma unroll
      for (int q = 0; q < kNMax / 4; ++q) {
        if (NF || 4 * q < N) {
          float a4[4], b4[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int n = 4 * q + i;
            const float apn = cst[0][n];
            const float a = exp2_hw(dl * apn);
            float bu;
            if (FORM == 0) {
              bu = dl * Bv[n] * x;
            } else if (FORM == 1 || ((fast_mask >> n) & 1)) {
              const float wu = x * Bv[n];
              bu = fmaf(a, wu, -wu);  // (abar - 1) u B, in g units
            } else {
              bu = dl * Bv[n] * zoh_phi(dl * apn * kLn2, a) * x;  // Delta A = Delta A log2(e) ln 2
            }
            a4[i] = rst ? 0.0f : a;
            b4[i] = bu;
          }
          pair_scan4(a4, b4);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            pa[4 * q + i] = a4[i];
            pb[4 * q + i] = b4[i];
          }
        }
      }
    };
    if (!ZOH) pairs(std::integral_constant<int, 0>());
    else if (all_fast) pairs(std::integral_constant<int, 1>());
    else pairs(std::integral_constant<int, 2>());
    const int par = (int)(ck & 1);
    if (lane == 63) {
#pragma unroll
      for (int n = 0; n < kNMax; ++n)
        if (NF || n < N) tot[par][w][n] = make_float2(pa[n], pb[n]);
    }
    lds_barrier();

    // (2) lane n: the carry into this wave's tokens, and into the next chunk
    float cin = carry;
    if (lane < N) {
      float cc = carry;
#pragma unroll
      for (int j = 0; j < kTW; ++j) {
        if (j == w) cin = cc;
        const float2 pj = tot[par][j][lane];
        cc = fmaf(pj.x, cc, pj.y);
      }
      carry = cc;
    }

    // (3) the states of this lane's token and the readout
    // the lane of the last token of a 16-token group writes the checkpoint of
    // the next group (the state before its first token), in h units
    const bool wck = CKPT && (t % 16 == 15) && t + 1 < L;
    float* ckp = ckpt + ((b * nck + (wck ? (t + 1) / 16 : 0)) * dim + c) * N;
    float acc = 0.0f;
#pragma unroll
    for (int n = 0; n < kNMax; ++n) {
      if (NF || n < N) {
        const float h = fmaf(pa[n], lane_bcast(cin, n), pb[n]);
        acc = fmaf(Cv[n] * cst[1][n] + (ZOH ? 0.0f : Cv[n]), h, acc);
        if (wck) ckp[n] = ZOH ? h * cst[1][n] : h;  // g / A where g is carried
      }
    }
    if (t < L) store_io(y + (b * L + t0) * dim + c + (uint32_t)tl0 * (uint32_t)dim,
                        live ? (acc + dskip * x) * gz : 0.0f);
  }

  if (last_state && w == 0 && lane < N)
    last_state[(b * dim + c) * N + lane] = fast_l ? carry * ca_l : carry;
}

// ---------------------------------------------------------------------------
// One wave per channel, or four channels per wave; four consecutive tokens
// per lane.
//
// For wide layers (many (batch, channel) rows) the time-parallel scan gives
// each row a segment of LPC lanes within one wave, so no carry crosses waves:
// LPC = 64 (one channel per wave) or 16 (four channels per wave, one per row
// of 16 lanes).  A block owns CPB consecutive channels of one batch entry, and
// each segment walks its channel's sequence in chunks of 4 LPC tokens, lane l
// of the segment holding tokens 4l .. 4l + 3.  Per state:
//   - the lane forms its four pairs and composes them in order (in-lane
//     prefix: three combine steps);
//   - the segment scans its LPC lane totals with DPP (pair_scan4 over the
//     wave, or its four in-row levels over rows of 16 lanes), so the scan
//     levels are paid once per four tokens;
//   - the carry enters through the segment's first lane (b = A_tot carry +
//     B_tot there; the other lanes read a zero carry), so after the scan each
//     lane's b is the state after its last token, he; a shift by one lane (DPP
//     wave_shr, or row_shr within rows; the segment's first lane keeping the
//     carry) gives the state before its first token; each token's state is
//     then one fma with its in-lane prefix, and the segment's last lane's he is
//     the next carry.
// Sixteen-lane segments skip the two scan levels that cross rows (one VALU
// instruction per update) and share each staged B and C row among twice as
// many channels, but make a quarter as many waves: the host takes them where
// the rows still give every SIMD three waves.
// Each chunk's inputs are staged in LDS by the whole block: u, Delta (after
// the softplus) and silu(z) as a (channel, token) tile read from global
// memory in row segments of the block's channels (a lane reading its own
// channel's four tokens would touch one cache line per element), and B and C
// as fp32 in the order the lanes read them, so a lane's read of four states of
// one of its tokens is one conflict-free 16-byte access.  Two barriers per
// chunk: after staging, and after the chunk's last read.
constexpr int kWT = 4;  // tokens per lane

template <int CPW>  // channels per wave: 1 or 4
struct WaveShape {
  static constexpr int LPC = 64 / CPW;          // lanes per channel
  static constexpr int WPB = CPW == 1 ? 8 : 4;  // waves per block
  static constexpr int CPB = WPB * CPW;         // channels per block
  static constexpr int TCK = LPC * kWT;         // tokens per chunk
  static constexpr int NT = 64 * WPB;           // threads per block
  static constexpr int TPT = CPB / 4;           // tile-staging threads per token (4 channels each)
  static constexpr int SPT = 16 * TCK / NT;     // B and C states per staging thread
  // waves per SIMD the registers are sized for: four (128 VGPRs) with one
  // channel per wave; three (168) with four, which the host picks only where
  // the layer has about three such waves per SIMD
  static constexpr int WPS = CPW == 1 ? 4 : 3;
  // Staged B and C: a reader's address is a constant plus 16 bytes times its
  // lane, and the writers in one pass of the LDS (16 lanes of 16 bytes) must
  // reach 16 different groups of 4 banks.  Rows are padded by ROW - LPC slots
  // and each state group's rows by QPAD: with one wave per channel a pass
  // holds tokens 0..7 (row offset i, slot l) of two groups two apart, at
  // group 2 i + l + 8 (q / 2); with four channels per wave, tokens 0..3 of
  // all four groups, at 4 i + q.
  static constexpr int ROW = LPC + (CPW == 1 ? 2 : 4);
  static constexpr int QPAD = CPW == 1 ? 4 : 1;
  // The (channel, token) tiles' rows are padded so that the staging threads of
  // one token, whose channel rows are 4 apart, write different banks: by 32
  // bytes (1 wave per channel: 2 threads per token) or 16 (4 channels per
  // wave: 4 threads per token).  Rows stay 16-byte aligned.
  static constexpr int XPAD = CPW == 1 ? 4 : 2;  // float2 slots
  static constexpr int GPAD = CPW == 1 ? 8 : 4;  // float slots
  static_assert(CPW == 1 || CPW == 4, "one or four channels per wave");
  static_assert(TCK * TPT == NT && TCK * (16 / SPT) == NT, "the staging threads cover the chunk");
};

template <int CPW>
struct WaveSmem {
  using S = WaveShape<CPW>;
  // per channel and group of four states: A log2(e), the readout weight, and
  // the carry (g units where fast), as three float4.  Slot 0 is read by the
  // segment's first lane, slot 1 (the same constants, a zero carry) by the
  // others: one pointer per lane reaches all three with immediate offsets
  // (first in the struct, so that the offsets fit the LDS instructions').
  float4 kq[S::CPB][kNMax / 4][2][3];
  // [state group][token in lane * ROW + lane in segment], QPAD spare slots
  // after each group's rows
  float4 b[kNMax / 4][kWT * S::ROW + S::QPAD];
  float4 c[kNMax / 4][kWT * S::ROW + S::QPAD];
  // per channel of the tile, one token per slot (rows padded: XPAD, GPAD)
  float2 xd[S::CPB][S::TCK + S::XPAD];  // (x, Delta)
  float gz[S::CPB][S::TCK + S::GPAD];   // silu(z)
  float yt[S::CPB][S::TCK + S::GPAD];   // y, stored by the block in row segments
};

// The scan of pair_scan4_b within rows of 16 lanes (its first four levels):
// lane i of a row ends with the composition of lanes 0..i of that row.
#define SSM66_STEP4(CTRL)                                         \
  "v_fmac_f32_dpp %0, %0, %4 " CTRL " bank_mask:0xf\n\t"        \
  "v_fmac_f32_dpp %1, %1, %5 " CTRL " bank_mask:0xf\n\t"        \
  "v_fmac_f32_dpp %2, %2, %6 " CTRL " bank_mask:0xf\n\t"        \
  "v_fmac_f32_dpp %3, %3, %7 " CTRL " bank_mask:0xf\n\t"        \
  "v_mul_f32_dpp %4, %4, %4 " CTRL " bank_mask:0xf\n\t"         \
  "v_mul_f32_dpp %5, %5, %5 " CTRL " bank_mask:0xf\n\t"         \
  "v_mul_f32_dpp %6, %6, %6 " CTRL " bank_mask:0xf\n\t"         \
  "v_mul_f32_dpp %7, %7, %7 " CTRL " bank_mask:0xf\n\t"
__device__ __forceinline__ void pair_scan4_b_rows(float (&a)[4], float (&b)[4]) {
  asm volatile("s_nop 1\n\t"
               SSM66_STEP4("row_shr:1 row_mask:0xf")
               SSM66_STEP4("row_shr:2 row_mask:0xf")
               SSM66_STEP4("row_shr:4 row_mask:0xf")
               "v_fmac_f32_dpp %0, %0, %4 row_shr:8 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %1, %1, %5 row_shr:8 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %2, %2, %6 row_shr:8 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %3, %3, %7 row_shr:8 row_mask:0xf bank_mask:0xf\n\t"
               "s_nop 1"
               : "+v"(b[0]), "+v"(b[1]), "+v"(b[2]), "+v"(b[3]),
                 "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]));
}
#undef SSM66_STEP4

// Arguments as for scan_tpar_kernel, plus ntiles = ceil(dim / CPB) channel
// tiles per batch entry and vec_io: dim is a multiple of CPB and u, delta, z
// and y are 16-byte aligned (tiles are read and y written in row segments of
// 4 channels); NF and CKPT likewise.  Four waves per SIMD (128 VGPRs) let
// blocks share a CU.
template <typename IO, bool ZOH, bool GATE, bool NF, bool CKPT, int CPW>
__global__ __launch_bounds__(WaveShape<CPW>::NT, WaveShape<CPW>::WPS) void scan_wave_kernel(
    const IO* __restrict__ u, const IO* __restrict__ dr, const float* __restrict__ Am,
    const IO* __restrict__ Bm, const IO* __restrict__ Cm, const float* __restrict__ Dm,
    const IO* __restrict__ zz, const float* __restrict__ bias_v, const float* h0,
    const int32_t* __restrict__ seq_lens, const uint8_t* __restrict__ reset,
    IO* __restrict__ y, float* last_state, float* __restrict__ ckpt, const int64_t L,
    const int64_t dim, const int N, const int64_t ntiles, const int softplus, const int vec_io) {
  using S = WaveShape<CPW>;
  constexpr int LPC = S::LPC, CPB = S::CPB, TCK = S::TCK;
  __shared__ WaveSmem<CPW> sm;

  // XCD-aware order: each XCD gets a contiguous run of channel tiles, which
  // share the 128-byte lines of u, Delta, z and y in its L2.
  const int64_t nblk = (int64_t)gridDim.x, bid = blockIdx.x;
  const int64_t logical = (nblk % 8 == 0) ? (bid % 8) * (nblk / 8) + bid / 8 : bid;
  const int64_t b = logical / ntiles, tile = logical - b * ntiles;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int sl = CPW == 1 ? lane : (lane & (LPC - 1));  // lane within its channel's segment
  const int ch = CPW == 1 ? w : w * CPW + lane / LPC;   // channel within the tile
  const int64_t c0 = tile * CPB;             // first channel of the tile
  const int64_t c = c0 + ch;                 // this segment's channel
  const bool cvalid = c < dim;               // uniform per segment; every wave stages and syncs
  const int64_t cc = cvalid ? c : dim - 1;   // loads of a padding segment stay in bounds

  // per-state constants, lane n of the segment holding state n's
  const float a_l = sl < N ? Am[cc * N + sl] : 0.0f;
  const bool fast_l = ZOH && fabsf(a_l) >= 0.5f;  // ZOH g form for this state
  const float ca_l = fast_l ? 1.0f / a_l : 0.0f;
  // the fast states of this lane's channel, bit n for state n
  const uint32_t fast_bits = (uint32_t)(__ballot(fast_l) >> (CPW == 1 ? 0 : lane - sl)) & 0xffffu;
  // every state of every channel of the wave takes the g form (uniform)
  const bool all_fast = ZOH && __ballot(sl < N && cvalid && !fast_l) == 0;
  const float dskip = Dm ? Dm[cc] : 0.0f;
  // this channel's constants and carry (g units where fast) to LDS, lane n of
  // the segment holding state n's; states past N are finite dummies (A = 0,
  // carry 0), never read out
  if (sl < kNMax) {
    float hv = 0.0f;
    if (h0 && sl < N) hv = h0[(b * dim + cc) * N + sl];
    float* s0 = (float*)&sm.kq[ch][sl / 4][0][0] + (sl & 3);
    float* s1 = (float*)&sm.kq[ch][sl / 4][1][0] + (sl & 3);
    const float a2 = a_l * kLog2e, w1 = fast_l ? ca_l : (ZOH ? 1.0f : 0.0f);
    s0[0] = a2; s1[0] = a2;
    s0[4] = w1; s1[4] = w1;
    s0[8] = fast_l ? a_l * hv : hv;
    s1[8] = 0.0f;
  }
  const float4* kp = &sm.kq[ch][0][sl == 0 ? 0 : 1][0];  // this lane's constants slot
  const int64_t nck = (L + 15) / 16;  // checkpoints per sequence (CKPT)
  int64_t Leff = L;
  if (seq_lens) {
    const int64_t sl_b = seq_lens[b];
    Leff = sl_b < 0 ? 0 : (sl_b < L ? sl_b : L);
  }
  const int64_t row0 = b * L;

  // ---- B and C staging: thread j stages token j / TPK of the chunk, states
  // SPT (j % TPK) .. + SPT - 1 (SPT / 4 groups of four): a wave reads
  // consecutive rows.  Token t = 4 l + i of group q goes to slot l of row
  // [q][i].  Tokens past L are clamped to L - 1; padding tokens stage
  // B = C = 0.
  constexpr int SPT = S::SPT;
  constexpr int TPK = 16 / SPT;
  const int st_t = tid / TPK, st_h = tid % TPK;
  const int st_i = st_t & (kWT - 1), st_l = st_t / kWT;
  // raw staging words: bf16 pairs (SPT / 2 words) or fp32 values (SPT words) per tensor
  constexpr int SW = sizeof(IO) == 2 ? SPT / 2 : SPT;
  uint32_t sb[SW], sc[SW];
  bool st_live = false;
  auto stage_load = [&](int64_t t0) {
    int64_t t = t0 + st_t;
    st_live = t < Leff;
    t = t < L ? t : L - 1;
    if constexpr (NF) {
      // the chunk's rows from a uniform base; this thread's byte offset in
      // them (token t - t0, states SPT st_h ..) is the same every full chunk
      typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
      typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;
      const char* bb = (const char*)(Bm + (row0 + t0) * 16);
      const char* cb = (const char*)(Cm + (row0 + t0) * 16);
      const uint32_t off = (uint32_t)((t - t0) * 16 + SPT * st_h) * (uint32_t)sizeof(IO);
      if constexpr (SW % 4 == 0) {
#pragma unroll
        for (int j = 0; j < SW / 4; ++j) {
          const u32x4 vb = *(const u32x4*)(bb + off + 16 * j);
          const u32x4 vc = *(const u32x4*)(cb + off + 16 * j);
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            sb[4 * j + k] = vb[k];
            sc[4 * j + k] = vc[k];
          }
        }
      } else {
        static_assert(SW == 2, "8-byte pieces");
        const u32x2 vb = *(const u32x2*)(bb + off);
        const u32x2 vc = *(const u32x2*)(cb + off);
        sb[0] = vb[0]; sb[1] = vb[1];
        sc[0] = vc[0]; sc[1] = vc[1];
      }
    } else {
#pragma unroll
      for (int j = 0; j < SW; ++j) {
        sb[j] = 0u;
        sc[j] = 0u;
      }
#pragma unroll
      for (int j = 0; j < SPT; ++j) {
        const int n = SPT * st_h + j;
        const int64_t e = (row0 + t) * N + (n < N ? n : N - 1);
        uint32_t vb = 0u, vc = 0u;
        if (n < N) {
          if constexpr (sizeof(IO) == 2) {
            vb = ((const uint16_t*)Bm)[e];
            vc = ((const uint16_t*)Cm)[e];
          } else {
            vb = __float_as_uint(((const float*)Bm)[e]);
            vc = __float_as_uint(((const float*)Cm)[e]);
          }
        }
        if constexpr (sizeof(IO) == 2) {
          sb[j / 2] |= vb << (16 * (j & 1));
          sc[j / 2] |= vc << (16 * (j & 1));
        } else {
          sb[j] = vb;
          sc[j] = vc;
        }
      }
    }
  };
  // element j (0..SPT-1) of the staged words, as fp32; 0 for padding tokens
  // (PAD: the chunk holds some)
  auto st_elem = [&](auto pad_tag, const uint32_t (&wv)[SW], int j) -> float {
    float v;
    if constexpr (sizeof(IO) == 2)
      v = __uint_as_float((j & 1) ? (wv[j >> 1] & 0xffff0000u) : (wv[j >> 1] << 16));
    else
      v = __uint_as_float(wv[j]);
    if constexpr (decltype(pad_tag)::value) v = st_live ? v : 0.0f;
    return v;
  };
  auto stage_store_as = [&](auto pad_tag) {
    auto st_elem_p = [&](const uint32_t (&wv)[SW], int j) { return st_elem(pad_tag, wv, j); };
#pragma unroll
    for (int q2 = 0; q2 < SPT / 4; ++q2) {
      const int q = (SPT / 4) * st_h + q2;
      sm.b[q][st_i * S::ROW + st_l] = make_float4(st_elem_p(sb, 4 * q2), st_elem_p(sb, 4 * q2 + 1),
                                        st_elem_p(sb, 4 * q2 + 2), st_elem_p(sb, 4 * q2 + 3));
      sm.c[q][st_i * S::ROW + st_l] = make_float4(st_elem_p(sc, 4 * q2), st_elem_p(sc, 4 * q2 + 1),
                                        st_elem_p(sc, 4 * q2 + 2), st_elem_p(sc, 4 * q2 + 3));
    }
  };

  // ---- the (channel, token) tile of u, raw Delta and z: thread j takes token
  // j / TPT and channels 4 (j % TPT) .. + 3 of the tile, one row segment per
  // tensor (vec_io), else element by element with channels clamped to dim.
  constexpr int TPT = S::TPT;
  const int xt = tid / TPT, xh = tid % TPT;
  float xbias[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int64_t chk = c0 + 4 * xh + k;
    xbias[k] = bias_v ? bias_v[chk < dim ? chk : dim - 1] : 0.0f;
  }
  constexpr int XW = sizeof(IO) == 2 ? 2 : 4;  // 32-bit words per 4 channels
  uint32_t xu[XW], xr[XW], xz[XW];
  bool x_live = false;
  // byte offset of this thread's row segment from the chunk's first element
  // (c0 of token t0): token xt, channels 4 xh ..; the same every full chunk.
  // The launch keeps TCK dim elements within 32 bits of bytes.
  const uint32_t xoff = ((uint32_t)xt * (uint32_t)dim + 4u * (uint32_t)xh) * (uint32_t)sizeof(IO);
  auto tile_load = [&](int64_t t0) {
    int64_t t = t0 + xt;
    x_live = t < Leff;
    t = t < L ? t : L - 1;
    if (vec_io) {
      // uniform base, 32-bit per-thread byte offset (of the clamped token)
      const int64_t cb0 = (row0 + t0) * dim + c0;
      const uint32_t off =
          ((uint32_t)(t - t0) * (uint32_t)dim + 4u * (uint32_t)xh) * (uint32_t)sizeof(IO);
      const char* ub = (const char*)(u + cb0) + off;
      const char* db = (const char*)(dr + cb0) + off;
      const char* zb = (const char*)(zz + cb0) + off;
      if constexpr (sizeof(IO) == 2) {
        typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;
        const u32x2 a = *(const u32x2*)ub, d = *(const u32x2*)db;
        xu[0] = a[0]; xu[1] = a[1]; xr[0] = d[0]; xr[1] = d[1];
        if constexpr (GATE) {
          const u32x2 g = *(const u32x2*)zb;
          xz[0] = g[0]; xz[1] = g[1];
        }
      } else {
        typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
        const u32x4 a = *(const u32x4*)ub, d = *(const u32x4*)db;
#pragma unroll
        for (int k = 0; k < 4; ++k) { xu[k] = a[k]; xr[k] = d[k]; }
        if constexpr (GATE) {
          const u32x4 g = *(const u32x4*)zb;
#pragma unroll
          for (int k = 0; k < 4; ++k) xz[k] = g[k];
        }
      }
    } else {
#pragma unroll
      for (int k = 0; k < XW; ++k) { xu[k] = 0u; xr[k] = 0u; xz[k] = 0u; }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int64_t chk = c0 + 4 * xh + k;
        const int64_t e = (row0 + t) * dim + (chk < dim ? chk : dim - 1);
        uint32_t vu, vr, vz = 0u;
        if constexpr (sizeof(IO) == 2) {
          vu = ((const uint16_t*)u)[e];
          vr = ((const uint16_t*)dr)[e];
          if constexpr (GATE) vz = ((const uint16_t*)zz)[e];
          xu[k / 2] |= vu << (16 * (k & 1));
          xr[k / 2] |= vr << (16 * (k & 1));
          xz[k / 2] |= vz << (16 * (k & 1));
        } else {
          vu = __float_as_uint(((const float*)u)[e]);
          vr = __float_as_uint(((const float*)dr)[e]);
          if constexpr (GATE) vz = __float_as_uint(((const float*)zz)[e]);
          xu[k] = vu; xr[k] = vr; xz[k] = vz;
        }
      }
    }
  };
  auto x_elem = [&](const uint32_t (&wv)[XW], int k) -> float {
    if constexpr (sizeof(IO) == 2)
      return __uint_as_float((k & 1) ? (wv[k >> 1] & 0xffff0000u) : (wv[k >> 1] << 16));
    else
      return __uint_as_float(wv[k]);
  };
  // Delta = softplus(raw + bias); padding tokens take x = Delta = 0, so their
  // pair is the identity whatever their inputs hold (PAD: the chunk holds some)
  auto tile_store_as = [&](auto pad_tag) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float v = x_elem(xr, k) + xbias[k];
      float dlt = softplus ? softplus_f(v) : v;
      float xv = x_elem(xu, k);
      if constexpr (decltype(pad_tag)::value) {
        dlt = x_live ? dlt : 0.0f;
        xv = x_live ? xv : 0.0f;
      }
      sm.xd[4 * xh + k][xt] = make_float2(xv, dlt);
      if constexpr (GATE) sm.gz[4 * xh + k][xt] = silu_f(x_elem(xz, k));
    }
  };

  // y of the chunk: thread j stores token j / TPT, channels 4 (j % TPT) .. + 3
  // of the tile (one row segment with vec_io); tokens past L are not stored.
  // Reads yt before the next chunk's barrier, which orders it before yt is
  // written again.
  auto y_store = [&](int64_t t0) {
    const int64_t t = t0 + xt;
    if (t >= L) return;
    const int64_t e0 = (row0 + t) * dim + c0 + 4 * xh;
    float v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = sm.yt[4 * xh + k][xt];
    if (vec_io) {
      char* yb = (char*)(y + (row0 + t0) * dim + c0) + xoff;  // uniform base + this thread's offset
      if constexpr (sizeof(IO) == 2) {
        typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;
        u32x2 o;
        o[0] = pack_bf16x2(v[0], v[1]);
        o[1] = pack_bf16x2(v[2], v[3]);
        *(u32x2*)yb = o;
      } else {
        *(float4*)yb = make_float4(v[0], v[1], v[2], v[3]);
      }
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (c0 + 4 * xh + k < dim) store_io(y + e0 + k, v[k]);
    }
  };

  const int64_t nchunks = (L + TCK - 1) / TCK;
  if (nchunks > 0) {
    tile_load(0);
    stage_load(0);
  }

  for (int64_t ck = 0; ck < nchunks; ++ck) {
    const int64_t t0 = ck * TCK;
    // staging (every wave finished reading the previous chunk before the
    // barrier that ended it), then the next chunk's loads into the freed
    // registers
    if (t0 + TCK <= Leff) {  // no padding token in the chunk (uniform)
      tile_store_as(std::false_type());
      stage_store_as(std::false_type());
    } else {
      tile_store_as(std::true_type());
      stage_store_as(std::true_type());
    }
    if (ck + 1 < nchunks) {
      tile_load(t0 + TCK);
      stage_load(t0 + TCK);
    }
    lds_barrier();

    const bool full = t0 + TCK <= Leff;  // every token of the chunk is real (uniform)
    float x[kWT], dl[kWT], gz[kWT], acc[kWT];
    bool live[kWT], rst[kWT];
    {
      const float4 v0 = *(const float4*)&sm.xd[ch][kWT * sl];
      const float4 v1 = *(const float4*)&sm.xd[ch][kWT * sl + 2];
      x[0] = v0.x; dl[0] = v0.y; x[1] = v0.z; dl[1] = v0.w;
      x[2] = v1.x; dl[2] = v1.y; x[3] = v1.z; dl[3] = v1.w;
      if constexpr (GATE) {
        const float4 g = *(const float4*)&sm.gz[ch][kWT * sl];
        gz[0] = g.x; gz[1] = g.y; gz[2] = g.z; gz[3] = g.w;
      } else {
#pragma unroll
        for (int i = 0; i < kWT; ++i) gz[i] = 1.0f;
      }
    }
#pragma unroll
    for (int i = 0; i < kWT; ++i) {
      live[i] = full || t0 + kWT * sl + i < Leff;
      rst[i] = false;
      acc[i] = 0.0f;
    }
    // document starts in this chunk (the same for every channel of the block)
    bool any_rst = false;
    if (reset) {
#pragma unroll
      for (int i = 0; i < kWT; ++i) {
        const int64_t t = t0 + kWT * sl + i;
        rst[i] = live[i] && reset[row0 + t] != 0;
      }
      any_rst = __ballot(rst[0] || rst[1] || rst[2] || rst[3]) != 0;
    }
    // the lane's first token starts a 16-token checkpoint group
    const int64_t tl = t0 + kWT * sl;
    const bool wck = CKPT && cvalid && (sl % 4 == 0) && tl < L;
    float* ckp = ckpt + ((b * nck + (wck ? tl / 16 : 0)) * dim + cc) * N;

    auto group = [&](auto form_tag, auto rst_tag, int q) {
      constexpr int FORM = decltype(form_tag)::value;
      constexpr bool RST = decltype(rst_tag)::value;
      const float4* kpq = kp + 6 * q;
      const float4 a24 = kpq[0], w14 = kpq[1], cin4 = kpq[2];  // cin4: the carry in the first lane, else 0
      const float a2v[4] = {a24.x, a24.y, a24.z, a24.w};
      const float w1v[4] = {w14.x, w14.y, w14.z, w14.w};
      const float cinv[4] = {cin4.x, cin4.y, cin4.z, cin4.w};
      float pa[kWT][4], pb[kWT][4];
#pragma unroll
      for (int i = 0; i < kWT; ++i) {
        const float4 bv4 = sm.b[q][i * S::ROW + sl];
        const float bv[4] = {bv4.x, bv4.y, bv4.z, bv4.w};
        const float dx = FORM == 0 ? dl[i] * x[i] : 0.0f;  // Euler: Delta u, once per token
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int n = 4 * q + k;
          const float a = exp2_hw(dl[i] * a2v[k]);
          float bu;
          if (FORM == 0) {
            bu = dx * bv[k];
          } else if (FORM == 1 || ((fast_bits >> n) & 1)) {
            const float wu = x[i] * bv[k];
            bu = fmaf(a, wu, -wu);  // (abar - 1) u B, in g units
          } else {
            bu = dl[i] * bv[k] * zoh_phi(dl[i] * a2v[k] * kLn2, a) * x[i];
          }
          pa[i][k] = (RST && rst[i]) ? 0.0f : a;
          pb[i][k] = bu;
        }
      }
      // C: read after the scan where registers are short (128), else before the
      // prefix, so that the prefix and the scan cover the read's latency
      float cv[kWT][4];
      auto read_c = [&]() {
#pragma unroll
        for (int i = 0; i < kWT; ++i) {
          const float4 cv4 = sm.c[q][i * S::ROW + sl];
          cv[i][0] = cv4.x; cv[i][1] = cv4.y; cv[i][2] = cv4.z; cv[i][3] = cv4.w;
        }
      };
      if constexpr (S::WPS != 4) read_c();
      // in-lane prefix: token i's pair becomes the composition of tokens 0..i
#pragma unroll
      for (int i = 1; i < kWT; ++i) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          pb[i][k] = fmaf(pa[i][k], pb[i - 1][k], pb[i][k]);
          pa[i][k] *= pa[i - 1][k];
        }
      }
      float ta[4] = {pa[kWT - 1][0], pa[kWT - 1][1], pa[kWT - 1][2], pa[kWT - 1][3]};
      float tb[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) tb[k] = fmaf(ta[k], cinv[k], pb[kWT - 1][k]);  // first lane: the carry enters
      if constexpr (LPC == 64)
        pair_scan4_b(ta, tb);
      else
        pair_scan4_b_rows(ta, tb);
      if constexpr (S::WPS == 4) read_c();
      float he[4], hck[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        he[k] = tb[k];  // after the lane's last token
        // the state before the lane's first token: the previous lane's he; the
        // segment's first lane (no source lane) keeps the carry
        constexpr int kShr1 = LPC == 64 ? 0x138 /* wave_shr:1 */ : 0x111 /* row_shr:1 */;
        const float hin = __int_as_float(__builtin_amdgcn_update_dpp(
            __float_as_int(cinv[k]), __float_as_int(he[k]), kShr1, 0xf, 0xf, false));
#pragma unroll
        for (int i = 0; i < kWT; ++i) {
          const float h = (i == kWT - 1) ? he[k] : fmaf(pa[i][k], hin, pb[i][k]);
          acc[i] = fmaf(ZOH ? cv[i][k] * w1v[k] : cv[i][k], h, acc[i]);  // Euler reads out h itself
        }
        hck[k] = ZOH ? hin * w1v[k] : hin;  // g / A where g is carried
      }
      // the checkpoint: one 16-byte store of the group's four states (the
      // 16-state path's rows are 64-byte aligned), else state by state
      if (CKPT && wck) {
        if constexpr (NF) {
          *(float4*)(ckp + 4 * q) = make_float4(hck[0], hck[1], hck[2], hck[3]);
        } else {
#pragma unroll
          for (int k = 0; k < 4; ++k)
            if (4 * q + k < N) ckp[4 * q + k] = hck[k];
        }
      }
      // the segment's last lane holds the state after the chunk: the next carry
      if (sl == LPC - 1) sm.kq[ch][q][0][2] = make_float4(he[0], he[1], he[2], he[3]);
    };
    // one group of four states at a time (a rolled loop keeps one group's
    // pairs live, not all sixteen states')
    auto groups = [&](auto form_tag) {
      const int ng = NF ? kNMax / 4 : (N + 3) / 4;
      if (any_rst) {
#pragma unroll 1
        for (int q = 0; q < ng; ++q) group(form_tag, std::true_type(), q);
      } else {
#pragma unroll 1
        for (int q = 0; q < ng; ++q) group(form_tag, std::false_type(), q);
      }
    };
    if (!ZOH) groups(std::integral_constant<int, 0>());
    else if (all_fast) groups(std::integral_constant<int, 1>());
    else groups(std::integral_constant<int, 2>());

    {
      float yv[kWT];
#pragma unroll
      for (int i = 0; i < kWT; ++i) yv[i] = live[i] ? (acc[i] + dskip * x[i]) * gz[i] : 0.0f;
      *(float4*)&sm.yt[ch][kWT * sl] = make_float4(yv[0], yv[1], yv[2], yv[3]);
    }
    lds_barrier();  // the chunk's LDS is free for the next one, and y is staged
    y_store(t0);
  }

  // the carried value and its readout weight from LDS (1/A where g = A h is
  // carried), so that no per-lane constant has to live through the loop
  if (cvalid && last_state && sl < N) {
    const float g = ((const float*)&sm.kq[ch][sl / 4][0][2])[sl & 3];
    const float w1 = ((const float*)&sm.kq[ch][sl / 4][0][1])[sl & 3];
    last_state[(b * dim + c) * N + sl] = ((fast_bits >> sl) & 1) ? g * w1 : g;
  }
}

template <typename IO, bool ZOH, bool GATE, int CPW>
hipError_t wave_launch(const ScanParams& p, hipStream_t stream) {
  using S = WaveShape<CPW>;
  const int64_t ntiles = (p.dim + S::CPB - 1) / S::CPB;
  const int64_t nblk = ntiles * p.batch;
  // 32-bit offsets: lanes' element offsets, and the staging's byte offsets
  // within a chunk of TCK tokens
  if (nblk > 0x7fffffff || S::TCK * p.dim * (int64_t)sizeof(IO) >= 0xffffffffLL) return hipErrorInvalidValue;
  // the 16-state path reads B and C rows and writes checkpoint rows as
  // 16-byte vectors
  const bool vec = p.N == kNMax && (uintptr_t)p.B % 16 == 0 && (uintptr_t)p.C % 16 == 0 &&
                   (uintptr_t)p.ckpt % 16 == 0;
  auto kern = vec ? (p.ckpt ? scan_wave_kernel<IO, ZOH, GATE, true, true, CPW>
                            : scan_wave_kernel<IO, ZOH, GATE, true, false, CPW>)
                  : (p.ckpt ? scan_wave_kernel<IO, ZOH, GATE, false, true, CPW>
                            : scan_wave_kernel<IO, ZOH, GATE, false, false, CPW>);
  // the (channel, token) tiles are read and y written in row segments of 4 channels
  const int vec_io = p.dim % S::CPB == 0 && (uintptr_t)p.u % 16 == 0 && (uintptr_t)p.delta % 16 == 0 &&
                     (uintptr_t)p.z % 16 == 0 && (uintptr_t)p.y % 16 == 0;
  hipLaunchKernelGGL(kern, dim3((unsigned)nblk), dim3(S::NT), 0, stream, (const IO*)p.u,
                     (const IO*)p.delta, p.A, (const IO*)p.B, (const IO*)p.C, p.D,
                     (const IO*)p.z, p.delta_bias, p.h0, p.seq_lens, p.reset, (IO*)p.y,
                     p.last_state, p.ckpt, p.L, p.dim, (int)p.N, ntiles, p.softplus, vec_io);
  return hipGetLastError();
}

template <typename IO, int CPW>
hipError_t wave_io(const ScanParams& p, bool zoh, bool gate, hipStream_t stream) {
  if (zoh)
    return gate ? wave_launch<IO, true, true, CPW>(p, stream) : wave_launch<IO, true, false, CPW>(p, stream);
  return gate ? wave_launch<IO, false, true, CPW>(p, stream) : wave_launch<IO, false, false, CPW>(p, stream);
}

template <typename IO, bool ZOH, bool GATE>
hipError_t tpar_launch(const ScanParams& p, hipStream_t stream) {
  const int64_t nblk = p.batch * p.dim;
  if (nblk > 0x7fffffff || kTT * p.dim >= 0x7fffffff) return hipErrorInvalidValue;
  // the 16-state path reads B and C rows as 16-byte vectors
  const bool vec = p.N == kNMax && (uintptr_t)p.B % 16 == 0 && (uintptr_t)p.C % 16 == 0;
  auto kern = vec ? (p.ckpt ? scan_tpar_kernel<IO, ZOH, GATE, true, true>
                            : scan_tpar_kernel<IO, ZOH, GATE, true, false>)
                  : (p.ckpt ? scan_tpar_kernel<IO, ZOH, GATE, false, true>
                            : scan_tpar_kernel<IO, ZOH, GATE, false, false>);
  hipLaunchKernelGGL(kern, dim3((unsigned)nblk), dim3(64 * kTW), 0, stream, (const IO*)p.u,
                     (const IO*)p.delta, p.A, (const IO*)p.B, (const IO*)p.C, p.D,
                     (const IO*)p.z, p.delta_bias, p.h0, p.seq_lens, p.reset, (IO*)p.y,
                     p.last_state, p.ckpt, p.L, p.dim, (int)p.N, p.softplus);
  return hipGetLastError();
}

template <typename IO>
hipError_t tpar_io(const ScanParams& p, bool zoh, bool gate, hipStream_t stream) {
  if (zoh) return gate ? tpar_launch<IO, true, true>(p, stream) : tpar_launch<IO, true, false>(p, stream);
  return gate ? tpar_launch<IO, false, true>(p, stream) : tpar_launch<IO, false, false>(p, stream);
}

}  // namespace

hipError_t launch_scan_tpar(const ScanParams& p, int io_dtype, bool zoh, bool gate,
                            hipStream_t stream) {
  if (p.N < 1 || p.N > kNMax) return hipErrorInvalidValue;
  if (io_dtype == 1) return tpar_io<bf16_bits>(p, zoh, gate, stream);
  return tpar_io<float>(p, zoh, gate, stream);
}

hipError_t launch_scan_wave(const ScanParams& p, int io_dtype, bool zoh, bool gate,
                            int channels_per_wave, hipStream_t stream) {
  if (p.N < 1 || p.N > kNMax) return hipErrorInvalidValue;
  // the common case of the 16-lane layout: eight tokens per lane (scan_wave8.hip)
  if (channels_per_wave == 4 && scan_wave8_fits(p, io_dtype)) return launch_scan_wave8(p, zoh, gate, stream);
  if (channels_per_wave == 4)
    return io_dtype == 1 ? wave_io<bf16_bits, 4>(p, zoh, gate, stream) : wave_io<float, 4>(p, zoh, gate, stream);
  if (channels_per_wave != 1) return hipErrorInvalidValue;
  return io_dtype == 1 ? wave_io<bf16_bits, 1>(p, zoh, gate, stream) : wave_io<float, 1>(p, zoh, gate, stream);
}

}  // namespace ssm66
