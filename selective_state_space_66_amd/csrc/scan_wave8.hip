// scan_wave8.hip -- the selective scan with time across lanes, eight tokens
// per lane (gfx950).
//
// "Mamba and selective state spaces" (zerotofrontier.app/ssm/mamba), "Selection
// breaks the convolution": the update h_t = abar_t h_{t-1} + bbar_t u_t is a
// first-order linear recurrence whose steps compose associatively,
//   (a1, b1) then (a2, b2)  =  (a2 a1, a2 b1 + b2),
// so a row of lanes can scan it in O(log) combine steps.
//
// The layout of scan_tpar.hip's 16-lane kernel (a row of 16 lanes per channel,
// four channels per wave, 16 channels per block, the carry kept in the row
// from chunk to chunk), with eight consecutive tokens per lane instead of
// four: the four DPP levels of the row scan and the state entering each lane
// are paid once per eight tokens, and a chunk is 128 tokens.  The states are
// taken four at a time (a rolled loop over the four state groups: one group's
// 8 x 4 pairs live, three waves per SIMD).  Per group: each lane composes its
// tokens' (abar, bbar u) pairs into its total (the b part token by token, the
// a part as one exponential of the lane's summed step, since the abar of one
// state are exponentials of the same A), the row scans the 16 lane totals (the
// chunk's carry entering at the first lane), and each lane walks its tokens
// again from the state before its first one, adding C.h into each token's
// output.
//
// This kernel takes the common case of the Mamba layers: bf16 io, N = 16, no
// lengths or document starts, a width that is a multiple of 16 and 16-byte
// aligned rows; scan_tpar.hip's kernel takes the rest.  CKPT (the training
// forward): the lanes whose first token is a multiple of 16 (the even lanes of
// a row) also write the state before it, in h units, as the backward reads it:
// ckpt[((b * ceil(L / 16) + t / 16) * dim + c) * 16 + n].
//
// The per-state forms are scan_tpar.hip's: exponential-Euler bbar u = Delta u B;
// ZOH on g = A h where |A| >= 1/2 (bbar u = (abar - 1) u B in g units, read
// out with weight 1/A), else bbar = Delta B phi(Delta A).
//
// Staging per chunk, through LDS: u and Delta (after the softplus) as a
// (channel, token) tile, read from global memory in 16-byte row segments of 8
// channels; z as it is read (token-major, bf16); B and C as fp32 in the order
// the lanes read them.  y leaves the same way as z arrives: each lane writes
// its tokens' outputs into a token-major bf16 tile, and the block stores it in
// row segments.  Two barriers per chunk.
#include <type_traits>

#include "ssm_device.h"
#include "ssm_launch.h"
#include "ssm_wave8.h"

namespace ssm66 {

namespace {

constexpr int kN8 = 16;            // states
constexpr int kTPL8 = 8;           // tokens per lane
constexpr int kLPC8 = 16;          // lanes per channel: one DPP row
constexpr int kTCK8 = kTPL8 * kLPC8;  // tokens per chunk
constexpr int kCPB8 = 16;          // channels per block (4 waves x 4 rows)
constexpr int kNT8 = 256;          // threads per block
// LDS padding (chosen with a bank model of these accesses): the B and C rows
// of one token-in-lane hold 16 lanes in 17 float4 slots, and each state group
// 4 more; the (u, Delta) row of a channel holds the pairs of tokens 2p, 2p + 1
// of lane l in float4 slot p * 17 + l, so the 16 lanes of a row read 64
// consecutive words for each p; the token rows of z and
// y 2 more bf16 (9 words a row: the lanes of a row, 8 tokens apart, then reach
// 8 different banks; the rows are written and read in words).
constexpr int kROW8 = kLPC8 + 1;
constexpr int kQPAD8 = 4;
constexpr int kZPAD8 = 2;

struct Wave8Smem {
  // per channel and group of four states: A log2(e), the readout weight, and
  // the carry (g units where fast), as three float4.  Slot 0 is read by the
  // row's first lane, slot 1 (the same constants, a zero carry) by the others.
  float4 kq[kCPB8][kN8 / 4][2][3];
  float4 b[kN8 / 4][kTPL8 * kROW8 + kQPAD8];  // [group][token in lane * kROW8 + lane]
  float4 c[kN8 / 4][kTPL8 * kROW8 + kQPAD8];
  float2 xd[kCPB8][kTPL8 * kROW8];            // (u, Delta): [channel][(pair * kROW8 + lane) * 2 + token & 1]
  uint16_t zt[kTCK8][kCPB8 + kZPAD8];         // z, raw bf16, per token and channel
  uint16_t yt[kTCK8][kCPB8 + kZPAD8];         // y, bf16, per token and channel
  float bias[kCPB8];                          // delta bias per channel
};

// The inclusive pair scan within each row of 16 lanes for four states, with
// DPP sources 1, 2, 4, 8 lanes to the left: one step composes the source lane's
// (earlier) pair into the lane's own, b <- a * b_src + b, a <- a * a_src, as
// v_fmac_f32 and v_mul_f32 with a DPP source operand; the last step updates b
// alone.  With bound_ctrl off a lane with no source lane in its row is not
// written (it keeps its pair).  A VALU write followed by a DPP read of the same
// VGPR needs two wait states: each state's write is separated from its DPP read
// by the other states' instructions, and the block's first and last reads wait.
#define SSM66_W8STEP4(CTRL)                                           \
  "v_fmac_f32_dpp %0, %0, %4 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
  "v_fmac_f32_dpp %1, %1, %5 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
  "v_fmac_f32_dpp %2, %2, %6 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
  "v_fmac_f32_dpp %3, %3, %7 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
  "v_mul_f32_dpp %4, %4, %4 " CTRL " row_mask:0xf bank_mask:0xf\n\t"  \
  "v_mul_f32_dpp %5, %5, %5 " CTRL " row_mask:0xf bank_mask:0xf\n\t"  \
  "v_mul_f32_dpp %6, %6, %6 " CTRL " row_mask:0xf bank_mask:0xf\n\t"  \
  "v_mul_f32_dpp %7, %7, %7 " CTRL " row_mask:0xf bank_mask:0xf\n\t"
__device__ __forceinline__ void row_scan4(float (&a)[4], float (&b)[4]) {
  asm volatile("s_nop 1\n\t"
               SSM66_W8STEP4("row_shr:1")
               SSM66_W8STEP4("row_shr:2")
               SSM66_W8STEP4("row_shr:4")
               "v_fmac_f32_dpp %0, %0, %4 row_shr:8 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %1, %1, %5 row_shr:8 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %2, %2, %6 row_shr:8 row_mask:0xf bank_mask:0xf\n\t"
               "v_fmac_f32_dpp %3, %3, %7 row_shr:8 row_mask:0xf bank_mask:0xf\n\t"
               "s_nop 1"
               : "+v"(b[0]), "+v"(b[1]), "+v"(b[2]), "+v"(b[3]),
                 "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]));
}
#undef SSM66_W8STEP4

// Arguments as scan_tpar.hip's wave kernel (bf16 io, N = 16, dim a multiple of
// 16, the row tensors and B, C 16-byte aligned); ntiles = dim / 16.
template <bool ZOH, bool GATE, bool CKPT>
__global__ __launch_bounds__(kNT8, 3) void scan_wave8_kernel(
    const bf16_bits* __restrict__ u, const bf16_bits* __restrict__ dr, const float* __restrict__ Am,
    const bf16_bits* __restrict__ Bm, const bf16_bits* __restrict__ Cm, const float* __restrict__ Dm,
    const bf16_bits* __restrict__ zz, const float* __restrict__ bias_v, const float* h0,
    bf16_bits* __restrict__ y, float* last_state, float* __restrict__ ckpt, const int64_t L, const int64_t dim,
    const int64_t ntiles, const int softplus) {
  __shared__ Wave8Smem sm;

  // XCD-aware order: each XCD gets a contiguous run of channel tiles, which
  // share the 128-byte lines of u, Delta, z and y in its L2
  const int64_t nblk = (int64_t)gridDim.x, bid = blockIdx.x;
  const int64_t logical = (nblk % 8 == 0) ? (bid % 8) * (nblk / 8) + bid / 8 : bid;
  const int64_t b = logical / ntiles, tile = logical - b * ntiles;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave_id = __builtin_amdgcn_readfirstlane(tid >> 6);
  // the row's channel in the tile and the lane in the row; for per-(channel,
  // state) work the same thread stands for (channel ch, state sl)
  const int ch = tid >> 4, sl = tid & (kLPC8 - 1);
  const int64_t c0 = tile * kCPB8, row0 = b * L;
  const int64_t cs0 = (b * dim + c0) * kN8;  // the tile's (channel, state) rows: thread (ch, n) at + tid

  // per-state constants
  const float a_l = Am[c0 * kN8 + tid];
  const bool fast_l = ZOH && fabsf(a_l) >= 0.5f;  // ZOH g form for this state
  // the fast states of this lane's channel, bit n for state n
  const uint32_t fast_bits = (uint32_t)(__ballot(fast_l) >> (lane - sl)) & 0xffffu;
  // every state of every channel of the wave takes the g form (uniform)
  const bool all_fast = ZOH && __ballot(!fast_l) == 0;
  const float dskip = Dm ? Dm[c0 + ch] : 0.0f;
  {
    const float hv = h0 ? h0[cs0 + tid] : 0.0f;
    float* s0 = (float*)&sm.kq[ch][sl >> 2][0][0] + (sl & 3);
    float* s1 = (float*)&sm.kq[ch][sl >> 2][1][0] + (sl & 3);
    const float a2 = a_l * kLog2e, w1 = fast_l ? 1.0f / a_l : (ZOH ? 1.0f : 0.0f);
    s0[0] = a2; s1[0] = a2;
    s0[4] = w1; s1[4] = w1;
    s0[8] = fast_l ? a_l * hv : hv;
    s1[8] = 0.0f;
  }
  if (tid < kCPB8) sm.bias[tid] = bias_v ? bias_v[c0 + tid] : 0.0f;
  lds_barrier();  // the constants and the bias, before the first staging reads them

  // ---- staging.  Addresses: a uniform base per chunk and a 32-bit byte
  // offset per thread (the launch keeps a chunk's rows within 32 bits).
  typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
  auto bf = [](uint32_t wv, int hi) { return __uint_as_float(hi ? (wv & 0xffff0000u) : (wv << 16)); };
  // the (channel, token) tile and z: thread (token xt, channels 8 xh .. + 7)
  const int xt = tid >> 1, xh = tid & 1;
  auto xoff = [&](int64_t t0) -> uint32_t {
    const int64_t tl = L - 1 - t0;
    const uint32_t tt = (uint32_t)(xt < tl ? (int64_t)xt : tl);
    return (tt * (uint32_t)dim + 8u * (uint32_t)xh) * 2u;
  };
  u32x4 xu, xr, xz;
  auto tile_load = [&](int64_t t0) {
    const int64_t cb = (row0 + t0) * dim + c0;
    const uint32_t off = xoff(t0);
    xu = *(const u32x4*)((const char*)(u + cb) + off);
    xr = *(const u32x4*)((const char*)(dr + cb) + off);
    if constexpr (GATE) xz = *(const u32x4*)((const char*)(zz + cb) + off);
  };
  // padding tokens (past L) take u = Delta = 0: their pair is the identity
  auto tile_store = [&](int64_t t0) {
    const bool live = t0 + xt < L;
    const int xslot = (((xt & (kTPL8 - 1)) >> 1) * kROW8 + (xt >> 3)) * 2 + (xt & 1);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float v = bf(xr[k >> 1], k & 1) + sm.bias[8 * xh + k];
      const float dl = softplus ? softplus_f(v) : v;
      sm.xd[8 * xh + k][xslot] = live ? make_float2(bf(xu[k >> 1], k & 1), dl) : make_float2(0.0f, 0.0f);
    }
    if constexpr (GATE) {
      uint32_t* zw = (uint32_t*)&sm.zt[xt][8 * xh];
#pragma unroll
      for (int j = 0; j < 4; ++j) zw[j] = xz[j];
    }
  };
  // B and C: thread (token st, states 8 sq .. + 7: groups 2 sq, 2 sq + 1),
  // stored where lane st / 8 reads its token st % 8
  const int st = tid >> 1, sq = tid & 1;
  u32x4 sb, sc;
  auto bc_load = [&](int64_t t0) {
    const int64_t tl = L - 1 - t0;
    const uint32_t tt = (uint32_t)(st < tl ? (int64_t)st : tl);
    const uint32_t off = (tt * kN8 + 8u * (uint32_t)sq) * 2u;
    const int64_t bb = (row0 + t0) * kN8;
    sb = *(const u32x4*)((const char*)(Bm + bb) + off);
    sc = *(const u32x4*)((const char*)(Cm + bb) + off);
  };
  auto bc_store = [&](int64_t t0) {
    const bool live = t0 + st < L;
    const int slot = (st & (kTPL8 - 1)) * kROW8 + (st >> 3);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float4 vb = make_float4(bf(sb[2 * j], 0), bf(sb[2 * j], 1), bf(sb[2 * j + 1], 0), bf(sb[2 * j + 1], 1));
      const float4 vc = make_float4(bf(sc[2 * j], 0), bf(sc[2 * j], 1), bf(sc[2 * j + 1], 0), bf(sc[2 * j + 1], 1));
      sm.b[2 * sq + j][slot] = live ? vb : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      sm.c[2 * sq + j][slot] = live ? vc : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
  };
  // y of the chunk: thread (token xt, channels 8 xh .. + 7), one row segment
  auto y_store = [&](int64_t t0) {
    if (t0 + xt >= L) return;
    const int64_t cb = (row0 + t0) * dim + c0;
    const uint32_t* yw = (const uint32_t*)&sm.yt[xt][8 * xh];
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = yw[j];
    *(u32x4*)((char*)(y + cb) + xoff(t0)) = o;
  };

  const int64_t nchunks = (L + kTCK8 - 1) / kTCK8;
  if (nchunks > 0) {
    tile_load(0);
    bc_load(0);
  }
  for (int64_t ck = 0; ck < nchunks; ++ck) {
    const int64_t t0 = ck * kTCK8;
    tile_store(t0);
    bc_store(t0);
    if (ck + 1 < nchunks) {
      tile_load(t0 + kTCK8);
      bc_load(t0 + kTCK8);
    }
    lds_barrier();

    // the lane's first token starts a 16-token checkpoint group (CKPT): its
    // row is the chunk's first (a uniform base) plus sl / 2 groups and the
    // channel (a 32-bit offset)
    const bool wck = CKPT && (sl % 2 == 0) && t0 + kTPL8 * sl < L;
    float* ckb = CKPT ? ckpt + ((b * ((L + 15) / 16) + t0 / 16) * dim + c0) * kN8 : nullptr;
    const uint32_t cko = ((uint32_t)(sl >> 1) * (uint32_t)dim + (uint32_t)ch) * kN8;

    float x[kTPL8], dl[kTPL8], acc[kTPL8];
#pragma unroll
    for (int j = 0; j < kTPL8 / 2; ++j) {
      const float4 v = *(const float4*)&sm.xd[ch][(j * kROW8 + sl) * 2];
      x[2 * j] = v.x; dl[2 * j] = v.y; x[2 * j + 1] = v.z; dl[2 * j + 1] = v.w;
    }
#pragma unroll
    for (int i = 0; i < kTPL8; ++i) acc[i] = 0.0f;
    // the lane's summed step: exp2(A log2(e) * dsum) is the product of its
    // eight abar, for every state
    float dsum = dl[0];
#pragma unroll
    for (int i = 1; i < kTPL8; ++i) dsum += dl[i];

    // this lane's constants slot (+ 6 q: group q), and its channel's carry
    // slots: formed here from the wave's index and the lane's (mbcnt), not
    // kept in registers through the staging
    const int lid = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    const int chk = wave_id * 4 + (lid >> 4);
    const float4* kp = &sm.kq[chk][0][(lid & 15) == 0 ? 0 : 1][0];
    float4* kcarry = &sm.kq[chk][0][0][2];  // + 6 q: group q

    // one group of four states at a time (a rolled loop)
    auto groups = [&](auto form_tag) {
      constexpr int FORM = decltype(form_tag)::value;  // 0 Euler, 1 ZOH all fast, 2 ZOH mixed
#pragma unroll 1
      for (int q = 0; q < kN8 / 4; ++q) {
        const float4 a24 = kp[6 * q], w14 = kp[6 * q + 1], cin4 = kp[6 * q + 2];
        const float a2v[4] = {a24.x, a24.y, a24.z, a24.w}, w1v[4] = {w14.x, w14.y, w14.z, w14.w};
        const float cinv[4] = {cin4.x, cin4.y, cin4.z, cin4.w};
        float pa[kTPL8][4], pb[kTPL8][4];
#pragma unroll
        for (int i = 0; i < kTPL8; ++i) {
          const float4 bv4 = sm.b[q][i * kROW8 + sl];
          const float bv[4] = {bv4.x, bv4.y, bv4.z, bv4.w};
          const float dx = FORM == 0 ? dl[i] * x[i] : 0.0f;  // Euler: Delta u, once per token
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const float a = exp2_hw(dl[i] * a2v[k]);
            float bu;
            if (FORM == 0) {
              bu = dx * bv[k];
            } else if (FORM == 1 || ((fast_bits >> (4 * q + k)) & 1)) {
              const float wu = x[i] * bv[k];
              bu = fmaf(a, wu, -wu);  // (abar - 1) u B, in g units
            } else {
              bu = dl[i] * bv[k] * zoh_phi(dl[i] * a2v[k] * kLn2, a) * x[i];
            }
            pa[i][k] = a;
            pb[i][k] = bu;
          }
        }
        // the lane's total pair: the b part composed token by token from a
        // zero state, the a part as one exponential of the summed step
        float ta[4], tb[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) tb[k] = pb[0][k];
#pragma unroll
        for (int i = 1; i < kTPL8; ++i) {
#pragma unroll
          for (int k = 0; k < 4; ++k) tb[k] = fmaf(pa[i][k], tb[k], pb[i][k]);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          ta[k] = exp2_hw(dsum * a2v[k]);
          tb[k] = fmaf(ta[k], cinv[k], tb[k]);  // first lane: the carry enters
        }
        row_scan4(ta, tb);
        float hin[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
          // the state before the lane's first token: the previous lane's
          // total; the row's first lane (no source lane) keeps the carry
          hin[k] = __int_as_float(__builtin_amdgcn_update_dpp(
              __float_as_int(cinv[k]), __float_as_int(tb[k]), 0x111 /* row_shr:1 */, 0xf, 0xf, false));
        // the checkpoint: g / A where g is carried, one 16-byte store
        if (CKPT && wck)
          *(float4*)(ckb + cko + 4 * q) = ZOH ? make_float4(hin[0] * w1v[0], hin[1] * w1v[1], hin[2] * w1v[2], hin[3] * w1v[3])
                                        : make_float4(hin[0], hin[1], hin[2], hin[3]);
        // the states after each token, from the state before the lane's first
#pragma unroll
        for (int i = 0; i < kTPL8; ++i) {
          const float4 cv4 = sm.c[q][i * kROW8 + sl];
          const float cv[4] = {cv4.x, cv4.y, cv4.z, cv4.w};
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            hin[k] = (i == kTPL8 - 1) ? tb[k] : fmaf(pa[i][k], hin[k], pb[i][k]);
            acc[i] = fmaf(ZOH ? cv[k] * w1v[k] : cv[k], hin[k], acc[i]);  // Euler reads out h itself
          }
        }
        // the row's last lane holds the state after the chunk: the next carry
        if (sl == kLPC8 - 1) kcarry[6 * q] = make_float4(tb[0], tb[1], tb[2], tb[3]);
      }
    };
    if (!ZOH) groups(std::integral_constant<int, 0>());
    else if (all_fast) groups(std::integral_constant<int, 1>());
    else groups(std::integral_constant<int, 2>());

    // y = (C.h + D u) silu(z) of the lane's tokens, into the token-major tile
#pragma unroll
    for (int i = 0; i < kTPL8; ++i) {
      float yv = fmaf(dskip, x[i], acc[i]);
      if constexpr (GATE) yv *= silu_f(__uint_as_float((uint32_t)sm.zt[kTPL8 * sl + i][ch] << 16));
      store_io(&sm.yt[kTPL8 * sl + i][ch], yv);
    }
    lds_barrier();  // the chunk's LDS is free for the next one, and y is staged
    y_store(t0);
  }

  // the carried value and its readout weight (1/A where g = A h is carried).
  // The thread index is formed again from the wave's index (a scalar) and the
  // lane's, so that no address for this step is kept in registers (or
  // scratch) across the chunk loop.
  if (last_state) {
    const int t = wave_id * 64 + (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    const float* kqs = (const float*)&sm.kq[t >> 4][(t & 15) >> 2][0][0] + (t & 3);
    const float g = kqs[8], w1 = kqs[4];
    const bool fast = ZOH && fabsf(Am[c0 * kN8 + t]) >= 0.5f;
    last_state[cs0 + t] = fast ? g * w1 : g;
  }
}

template <bool ZOH, bool GATE, bool CKPT>
hipError_t wave8_launch(const ScanParams& p, hipStream_t stream) {
  const int64_t ntiles = p.dim / kCPB8;
  const int64_t nblk = ntiles * p.batch;
  hipLaunchKernelGGL((scan_wave8_kernel<ZOH, GATE, CKPT>), dim3((unsigned)nblk), dim3(kNT8), 0, stream,
                     (const bf16_bits*)p.u, (const bf16_bits*)p.delta, p.A, (const bf16_bits*)p.B,
                     (const bf16_bits*)p.C, p.D, (const bf16_bits*)p.z, p.delta_bias, p.h0, (bf16_bits*)p.y,
                     p.last_state, p.ckpt, p.L, p.dim, ntiles, p.softplus);
  return hipGetLastError();
}

}  // namespace

bool scan_wave8_fits(const ScanParams& p, int io_dtype) {
  auto al16 = [](const void* ptr) { return ptr == nullptr || (uintptr_t)ptr % 16 == 0; };
  return io_dtype == 1 && p.N == kN8 && p.dim % kCPB8 == 0 && !p.seq_lens && !p.reset && al16(p.ckpt) &&
         al16(p.u) && al16(p.delta) && al16(p.z) && al16(p.y) && al16(p.B) && al16(p.C) &&
         p.batch * (p.dim / kCPB8) <= 0x7fffffff && kTCK8 * p.dim * 2 < 0xffffffffLL;
}

hipError_t launch_scan_wave8(const ScanParams& p, bool zoh, bool gate, hipStream_t stream) {
  if (p.ckpt) {
    if (zoh) return gate ? wave8_launch<true, true, true>(p, stream) : wave8_launch<true, false, true>(p, stream);
    return gate ? wave8_launch<false, true, true>(p, stream) : wave8_launch<false, false, true>(p, stream);
  }
  if (zoh) return gate ? wave8_launch<true, true, false>(p, stream) : wave8_launch<true, false, false>(p, stream);
  return gate ? wave8_launch<false, true, false>(p, stream) : wave8_launch<false, false, false>(p, stream);
}

}  // namespace ssm66
