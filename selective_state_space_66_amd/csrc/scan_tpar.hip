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
#undef SSM66_STEP4

__device__ __forceinline__ float lane_bcast(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// Pointers are separate __restrict__ arguments; y must not overlap any input,
// and last_state none but h0 (read before the first chunk, written after the
// last).
// NF: N == 16, whose B and C rows are read as 16-byte vectors.  CKPT: also
// write the state before every 16th token to ckpt (batch, ceil(L / 16), dim, N).
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

template <typename IO, bool ZOH, bool GATE>
hipError_t tpar_launch(const ScanParams& p, hipStream_t stream) {
  const int64_t nblk = p.batch * p.dim;
  if (nblk > 0x7fffffff || kTT * p.dim >= 0x7fffffff) return hipErrorInvalidValue;
  auto kern = p.N == kNMax ? (p.ckpt ? scan_tpar_kernel<IO, ZOH, GATE, true, true>
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

}  // namespace ssm66
