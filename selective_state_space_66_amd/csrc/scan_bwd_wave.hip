// scan_bwd_wave.hip -- the backward pass of the selective scan with time
// across lanes (gfx950): rows of 16 lanes, as in the forward's 16-lane kernel.
//
// "Mamba and selective state spaces" (zerotofrontier.app/ssm/mamba), "Why the
// scan must be fused": the backward pass reloads the inputs, recomputes the
// states on chip and runs the recurrence's adjoint backwards.  With
// ds_t = dy_t silu(z_t), the adjoint of h_t,
//   q_t = ds_t C_t + abar_{t+1} q_{t+1},
// is itself a first-order linear recurrence, run from the last token to the
// first, and ("Selection breaks the convolution") composing two of its steps
// is associative: it takes the same pair scan as the state, with the order of
// the lanes reversed.
//
// This kernel takes the ZOH blocks whose states all have |A| >= 1/2, in the
// forward's g form (g = A h, g_t = abar_t (g_{t-1} + u_t B_t) - u_t B_t).
// Per update, with s_t = g_{t-1} + u_t B_t and w_t = q_t (abar_t - 1) / A:
//   dDelta_t += q_t abar_t s_t        (d h_t / d Delta = abar (A h_{t-1} + u B))
//   dB_t += w_t u_t, du_t += w_t B_t  (bbar u = (abar - 1) u B / A)
//   dC_t += ds_t h_t, and the readout C_t . h_t (for dz)
//   A dA += Delta_t q_t abar_t s_t - ds_t C_t h_t.
// The last line is d h_t / dA = Delta abar s / A - bbar u / A summed against
// q, with the sum over the updates of q_t bbar_t u_t replaced by
// sum_t ds_t C_t h_t + dlast h_T - h0 dh0 (the adjoint identity of a linear
// recurrence): no phi' is needed.  h_T, the state after the last real token,
// and h0 dh0 enter once.
//
// Layout.  A block owns one batch entry and 16 channels (4 waves, 4 channels
// per wave, a row of 16 lanes per channel) and walks the sequence in chunks of
// 64 tokens from the last to the first; lane l of a row takes tokens
// 4 l .. 4 l + 3 of the chunk.  Per group of four states:
//   1. the state: each lane composes its tokens' (abar, bbar u) pairs, the row
//      scans its 16 lane totals with DPP row shifts to the right (the chunk's
//      checkpoint entering at the first lane), and each lane recovers the
//      state after each of its tokens;
//   2. the adjoint: each lane composes its tokens' adjoint pairs from its last
//      token down, the row scans them with DPP row shifts to the left (the
//      adjoint from the chunk after entering at the last lane), and each lane
//      recovers q at each of its tokens; the first lane's result is the
//      adjoint carried into the chunk before;
//   3. the gradients above.  Sums over the states of one (token, channel) --
//      dDelta, du, the readout -- stay in the lane.  dB and dC, sums over
//      channels, are added across the wave's four rows with permlane swaps
//      (each swap step halves the values a lane holds) and across the block's
//      four waves in LDS, leaving one partial per 16-channel tile, as the other
//      backward kernel writes them.
// Without the forward's checkpoints a first sweep runs step 1 through the
// sequence and writes the state at every chunk start.
//
// Padding past a sequence's length is staged as u = Delta = dy = 0: its pairs
// are the identity and its gradients zero.
#include <type_traits>

#include "ssm_bwd.h"
#include "ssm_device.h"

namespace ssm66 {

namespace {

constexpr int kN = 16;              // states (the only size this kernel takes)
constexpr int kTPL = 4;             // tokens per lane
constexpr int kLPC = 16;            // lanes per channel: one DPP row
constexpr int kTCK = kTPL * kLPC;   // tokens per chunk
constexpr int kCPB = 16;            // channels per block (4 waves x 4 rows)
constexpr int kNT = 256;            // threads per block
constexpr int kCkTok = 16;          // tokens per checkpoint interval
// LDS padding, as in the forward's 16-lane layout: each token-in-lane row of
// B and C holds 16 lanes in 20 float4 slots and each state group one spare
// slot, so that the lanes' 16-byte reads and the staging threads' writes fall
// on different banks; the (channel, token) rows are padded by 16 bytes.
constexpr int kROW = kLPC + 4;
constexpr int kQPAD = 1;
constexpr int kXPAD = 2;  // float2 slots
constexpr int kGPAD = 4;  // float slots
static_assert(kTCK % kCkTok == 0, "chunks start on checkpoints");

struct BWSmem {
  // per channel, group of four states and slot: A log2(e), 1/A, the state
  // entering the chunk (g units) and the adjoint entering it from the chunk
  // after.  Slot 0 holds the carries, read by the row's first lane (state)
  // and last lane (adjoint); slot 1 the same constants with zero carries, read
  // by the other lanes.
  float4 kq[kCPB][kN / 4][2][4];
  union {
    struct {
      float4 b[kN / 4][kTPL * kROW + kQPAD];  // [group][token in lane * kROW + lane]
      float4 c[kN / 4][kTPL * kROW + kQPAD];
      float2 xd[kCPB][kTCK + kXPAD];          // (u, Delta) per channel and token
    } in;
    struct {  // per (channel, token) sums, written after the chunk's last read of `in`
      float ddt[kCPB][kTCK + kGPAD];
      float dx[kCPB][kTCK + kGPAD];
      float sv[kCPB][kTCK + kGPAD];
    } out;
  } io;
  float ds[kCPB][kTCK + kGPAD];  // dy silu(z) per channel and token
  float cst[2][kCPB];            // D, delta bias per channel
  float dacc[kCPB][kN];          // A dA per (channel, state), summed over the chunks so far
  // dB and dC of one state group, per wave: [dB or dC][token][state in
  // group]; two buffers, so that one barrier per group orders the writes and
  // the reads
  float part[2][4][2 * kTCK * 4];
};

// The inclusive pair scan within each row of 16 lanes, four states at once,
// with DPP sources SHIFT:1, 2, 4, 8 lanes away: one step composes the source
// lane's pair into the lane's own,
//   b <- a * b_src + b,  a <- a * a_src,
// as v_fmac_f32 and v_mul_f32 with a DPP source operand; the last step updates
// b alone.  With bound_ctrl off, a lane with no source lane in its row is not
// written, i.e. it keeps its pair.  row_shr (sources to the left) composes
// earlier lanes first: lane i ends with lanes 0..i.  row_shl (sources to the
// right) composes later lanes: lane i ends with lanes i..15, the form of the
// adjoint, whose pair maps what comes from the right to what leaves to the
// left.  A VALU write followed by a DPP read of the same VGPR needs two wait
// states: each state's write is separated from its DPP read by the three other
// states' instructions, and the block's first and last reads wait.
#define SSM66_BSTEP4(CTRL)                                        \
  "v_fmac_f32_dpp %0, %0, %4 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
  "v_fmac_f32_dpp %1, %1, %5 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
  "v_fmac_f32_dpp %2, %2, %6 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
  "v_fmac_f32_dpp %3, %3, %7 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
  "v_mul_f32_dpp %4, %4, %4 " CTRL " row_mask:0xf bank_mask:0xf\n\t"  \
  "v_mul_f32_dpp %5, %5, %5 " CTRL " row_mask:0xf bank_mask:0xf\n\t"  \
  "v_mul_f32_dpp %6, %6, %6 " CTRL " row_mask:0xf bank_mask:0xf\n\t"  \
  "v_mul_f32_dpp %7, %7, %7 " CTRL " row_mask:0xf bank_mask:0xf\n\t"
#define SSM66_BLAST4(CTRL)                                        \
  "v_fmac_f32_dpp %0, %0, %4 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
  "v_fmac_f32_dpp %1, %1, %5 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
  "v_fmac_f32_dpp %2, %2, %6 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
  "v_fmac_f32_dpp %3, %3, %7 " CTRL " row_mask:0xf bank_mask:0xf\n\t"
__device__ __forceinline__ void row_scan_right(float (&a)[4], float (&b)[4]) {
  asm volatile("s_nop 1\n\t"
               SSM66_BSTEP4("row_shr:1")
               SSM66_BSTEP4("row_shr:2")
               SSM66_BSTEP4("row_shr:4")
               SSM66_BLAST4("row_shr:8")
               "s_nop 1"
               : "+v"(b[0]), "+v"(b[1]), "+v"(b[2]), "+v"(b[3]),
                 "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]));
}
// The same for two states (a group of four split in halves, half the
// registers): each state's write and its DPP read are three instructions apart.
#define SSM66_BSTEP2(CTRL)                                        \
  "v_fmac_f32_dpp %0, %0, %2 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
  "v_fmac_f32_dpp %1, %1, %3 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
  "v_mul_f32_dpp %2, %2, %2 " CTRL " row_mask:0xf bank_mask:0xf\n\t"  \
  "v_mul_f32_dpp %3, %3, %3 " CTRL " row_mask:0xf bank_mask:0xf\n\t"
#define SSM66_BLAST2(CTRL)                                        \
  "v_fmac_f32_dpp %0, %0, %2 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
  "v_fmac_f32_dpp %1, %1, %3 " CTRL " row_mask:0xf bank_mask:0xf\n\t"
__device__ __forceinline__ void row_scan_right(float (&a)[2], float (&b)[2]) {
  asm volatile("s_nop 1\n\t"
               SSM66_BSTEP2("row_shr:1")
               SSM66_BSTEP2("row_shr:2")
               SSM66_BSTEP2("row_shr:4")
               SSM66_BLAST2("row_shr:8")
               "s_nop 1"
               : "+v"(b[0]), "+v"(b[1]), "+v"(a[0]), "+v"(a[1]));
}
__device__ __forceinline__ void row_scan_left(float (&a)[2], float (&b)[2]) {
  asm volatile("s_nop 1\n\t"
               SSM66_BSTEP2("row_shl:1")
               SSM66_BSTEP2("row_shl:2")
               SSM66_BSTEP2("row_shl:4")
               SSM66_BLAST2("row_shl:8")
               "s_nop 1"
               : "+v"(b[0]), "+v"(b[1]), "+v"(a[0]), "+v"(a[1]));
}
#undef SSM66_BSTEP4
#undef SSM66_BLAST4
#undef SSM66_BSTEP2
#undef SSM66_BLAST2

// src from the lane one to the left (CTRL row_shr:1) or right (row_shl:1) in
// the row; the lane with no such neighbour gets old
template <int CTRL>
__device__ __forceinline__ float row_shift1(float old, float src) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(src), CTRL, 0xf,
                                                    0xf, false));
}
constexpr int kRowShr1 = 0x111;
constexpr int kRowShl1 = 0x101;

// Sums across rows of a wave.  permlane32_swap exchanges the upper 32 lanes of
// its first operand with the lower 32 lanes of its second: x + y afterwards is
// x summed over the two halves (rows r and r + 2) in the lower half and y
// summed in the upper one.  permlane16_swap exchanges the odd rows of its first
// operand with the even rows of its second: x + y is x summed over rows 2k and
// 2k + 1 in the even rows and y in the odd ones.
__device__ __forceinline__ float sum_halves(float x, float y) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_row_pairs(float x, float y) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Arguments and workspace as for scan_bwd_kernel (ssm_bwd.h); N = 16, dim a
// multiple of 16, no document starts, the (token, channel) tensors and B, C
// 16-byte aligned.  Three blocks share a CU (47 KB of LDS, registers for three
// waves per SIMD).
template <typename IO, bool GATE>
__global__ __launch_bounds__(kNT, 3) void scan_bwd_wave_kernel(const BwdArgs p) {
  __shared__ BWSmem sm;
  const IO* __restrict__ u = (const IO*)p.u;
  const IO* __restrict__ dr = (const IO*)p.delta;
  const IO* __restrict__ Bm = (const IO*)p.B;
  const IO* __restrict__ Cm = (const IO*)p.C;
  const IO* __restrict__ zz = (const IO*)p.z;
  const IO* __restrict__ dyp = (const IO*)p.dy;
  const int64_t L = p.L, dim = p.dim;

  // XCD-aware order: a batch entry's tiles run on one XCD and share its L2
  const int64_t nblk = (int64_t)gridDim.x, bid = blockIdx.x;
  const int64_t logical = (nblk % 8 == 0) ? (bid % 8) * (nblk / 8) + bid / 8 : bid;
  const int64_t b = logical / p.ntiles, tile = logical - b * p.ntiles;
  const int64_t c0 = tile * kCPB, row0 = b * L;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // the row's channel in the tile and the lane in the row; for per-(channel,
  // state) work the same thread stands for (channel ch, state sl)
  const int ch = tid >> 4, sl = tid & (kLPC - 1);
  int64_t Lb = L;  // real tokens of this sequence
  if (p.seq_lens) {
    const int64_t s = p.seq_lens[b];
    Lb = s < 0 ? 0 : (s < L ? s : L);
  }

  // every state of the tile with |A| >= 1/2, or the other kernel takes it
  const float a_n = p.A[c0 * kN + tid];
  if (__syncthreads_or(!(fabsf(a_n) >= 0.5f))) return;
  const float ca_n = 1.0f / a_n;
  {
    float* s0 = (float*)&sm.kq[ch][sl >> 2][0][0] + (sl & 3);
    float* s1 = (float*)&sm.kq[ch][sl >> 2][1][0] + (sl & 3);
    const float a2 = a_n * kLog2e;
    s0[0] = a2; s1[0] = a2;
    s0[4] = ca_n; s1[4] = ca_n;
    s0[8] = p.h0 ? p.h0[(b * dim + c0) * kN + tid] * a_n : 0.0f;  // the state entering the sequence
    s1[8] = 0.0f;
    s0[12] = p.dlast ? p.dlast[(b * dim + c0) * kN + tid] : 0.0f;  // the adjoint entering the last token
    s1[12] = 0.0f;
  }
  if (tid < kCPB) {
    sm.cst[0][tid] = p.D ? p.D[c0 + tid] : 0.0f;
    sm.cst[1][tid] = p.bias ? p.bias[c0 + tid] : 0.0f;
  }
  lds_barrier();
  const float4* kpf = &sm.kq[ch][0][sl == 0 ? 0 : 1][0];         // + 8 q: group q
  const float4* kpr = &sm.kq[ch][0][sl == kLPC - 1 ? 0 : 1][0];

  // ---- staging.  The (channel, token) tile: thread (token xt, channels
  // 4 xh .. 4 xh + 3), one row segment per tensor.  B and C: thread (token
  // st, states 4 sq .. 4 sq + 3), stored where lane st / 4 reads its token
  // st % 4.  Loads go to registers a chunk ahead.
  constexpr int XW = sizeof(IO) == 2 ? 2 : 4;  // 32-bit words per 4 elements
  typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;
  typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
  auto load4 = [](const IO* ptr, uint32_t (&wv)[XW]) {
    if constexpr (XW == 2) {
      const u32x2 v = *(const u32x2*)ptr;
      wv[0] = v[0]; wv[1] = v[1];
    } else {
      const u32x4 v = *(const u32x4*)ptr;
#pragma unroll
      for (int k = 0; k < 4; ++k) wv[k] = v[k];
    }
  };
  auto store4 = [](IO* ptr, const float (&v)[4]) {
    if constexpr (XW == 2) {
      u32x2 o;
      o[0] = pack_bf16x2(v[0], v[1]);
      o[1] = pack_bf16x2(v[2], v[3]);
      *(u32x2*)ptr = o;
    } else {
      *(float4*)ptr = make_float4(v[0], v[1], v[2], v[3]);
    }
  };
  auto elem = [](const uint32_t (&wv)[XW], int k) -> float {
    if constexpr (XW == 2)
      return __uint_as_float((k & 1) ? (wv[k >> 1] & 0xffff0000u) : (wv[k >> 1] << 16));
    else
      return __uint_as_float(wv[k]);
  };

  // Addresses: a uniform base per chunk (scalar registers) and a 32-bit byte
  // offset per thread (the launch keeps a chunk's rows within 32 bits).
  const int xt = tid >> 2, xh = tid & 3;
  // this thread's row segment from the chunk's first element (token t0,
  // channel c0), its token clamped into the sequence
  auto xoff = [&](int64_t t0) -> uint32_t {
    const int64_t tl = L - 1 - t0;
    const uint32_t tt = (uint32_t)(xt < tl ? (int64_t)xt : tl);
    return (tt * (uint32_t)dim + 4u * (uint32_t)xh) * (uint32_t)sizeof(IO);
  };
  auto at = [](const IO* base, uint32_t off) { return (const IO*)((const char*)base + off); };
  uint32_t xu[XW], xr[XW], xz[XW], xy[XW];
  auto tile_load = [&](int64_t t0, auto bwd_tag) {
    constexpr bool BWD = decltype(bwd_tag)::value;
    const int64_t cb = (row0 + t0) * dim + c0;
    const uint32_t off = xoff(t0);
    load4(at(u + cb, off), xu);
    load4(at(dr + cb, off), xr);
    if constexpr (BWD) {
      if constexpr (GATE) load4(at(zz + cb, off), xz);
      load4(at(dyp + cb, off), xy);
    }
  };
  // Staging the backward's chunk also takes what its epilogue needs for the
  // same (token, 4 channels) -- the thread that stages them finishes them --
  // so that the raw inputs are read and the transcendentals taken once:
  // softplus'(v), ds D, dy silu'(z) and dy silu'(z) D u; and it adds ds u
  // into the sums for dD.
  float ep_sg[4], ep_dsD[4], ep_dyg[4], ep_dyx[4];
  float accD[4] = {0.0f, 0.0f, 0.0f, 0.0f}, accB[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  auto tile_store = [&](int64_t t0, auto bwd_tag) {
    constexpr bool BWD = decltype(bwd_tag)::value;
    const bool live = t0 + xt < Lb;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int cl = 4 * xh + k;
      const float v = elem(xr, k) + sm.cst[1][cl];
      const float xv = live ? elem(xu, k) : 0.0f;
      if constexpr (!BWD) {
        const float dl = live ? (p.softplus ? softplus_f(v) : v) : 0.0f;
        sm.io.in.xd[cl][xt] = make_float2(xv, dl);
      } else {
        // softplus(v) = max(v, 0) + log(1 + e^-|v|) (as softplus_f) and its
        // derivative sigma(v) = (v >= 0 ? 1 : e^-|v|) / (1 + e^-|v|), from
        // one exponential
        float dl = v, sgv = 1.0f;
        if (p.softplus) {
          const float e = exp2_hw(-fabsf(v) * kLog2e);
          const float wv = 1.0f + e;
          const float r = (wv - 1.0f) - e;
          dl = fmaf(log2_hw(wv), kLn2, fmaxf(v, 0.0f) - r);
          sgv = (v >= 0.0f ? 1.0f : e) * rcp_hw(wv);
        }
        sm.io.in.xd[cl][xt] = make_float2(xv, live ? dl : 0.0f);
        const float dyv = live ? elem(xy, k) : 0.0f;
        float gz = 1.0f, dg = 0.0f;
        if constexpr (GATE) {
          const float zv = elem(xz, k);
          const float sz = rcp_hw(1.0f + exp2_hw(-zv * kLog2e));  // sigma(z)
          gz = zv * sz;                                          // silu(z)
          dg = sz * fmaf(zv, 1.0f - sz, 1.0f);                   // silu'(z)
        }
        const float d = dyv * gz;
        const float dskip = sm.cst[0][cl];
        sm.ds[cl][xt] = d;
        ep_sg[k] = live ? sgv : 0.0f;  // padding: no step size
        ep_dsD[k] = d * dskip;
        ep_dyg[k] = dyv * dg;
        ep_dyx[k] = ep_dyg[k] * dskip * xv;
        accD[k] = fmaf(d, xv, accD[k]);
      }
    }
  };
  const int st = tid >> 2, sq = tid & 3;
  uint32_t sb[XW], sc[XW];
  auto bc_load = [&](int64_t t0, auto bwd_tag) {
    const int64_t tl = L - 1 - t0;
    const uint32_t tt = (uint32_t)(st < tl ? (int64_t)st : tl);
    const uint32_t off = (tt * kN + 4u * (uint32_t)sq) * (uint32_t)sizeof(IO);
    const int64_t bb = (row0 + t0) * kN;
    load4(at(Bm + bb, off), sb);
    if constexpr (decltype(bwd_tag)::value) load4(at(Cm + bb, off), sc);
  };
  auto bc_store = [&](int64_t t0, auto bwd_tag) {
    const bool live = t0 + st < Lb;
    const int slot = (st & (kTPL - 1)) * kROW + (st >> 2);
    sm.io.in.b[sq][slot] = live ? make_float4(elem(sb, 0), elem(sb, 1), elem(sb, 2), elem(sb, 3))
                                : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if constexpr (decltype(bwd_tag)::value)
      sm.io.in.c[sq][slot] = live ? make_float4(elem(sc, 0), elem(sc, 1), elem(sc, 2), elem(sc, 3))
                                  : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  };
  // this lane's tokens: u and Delta
  auto read_xd = [&](float (&x)[kTPL], float (&dl)[kTPL]) {
    const float4 v0 = *(const float4*)&sm.io.in.xd[ch][kTPL * sl];
    const float4 v1 = *(const float4*)&sm.io.in.xd[ch][kTPL * sl + 2];
    x[0] = v0.x; dl[0] = v0.y; x[1] = v0.z; dl[1] = v0.w;
    x[2] = v1.x; dl[2] = v1.y; x[3] = v1.z; dl[3] = v1.w;
  };
  // step 1 for GW states (4 h0s .. of group q): the lane's pairs (pa, pb:
  // prefixes over its tokens, g units), composed into the lane total and
  // scanned over the row with the carry (cin, nonzero in the first lane only);
  // returns the total in (ta, tb): tb is the state after the lane's last token
  auto forward_pairs = [&](auto gw_tag, int q, int h0s, const float (&x)[kTPL], const float (&dl)[kTPL],
                           const float* a2v, const float* cinv, float (&ar)[kTPL][decltype(gw_tag)::value],
                           float (&pa)[kTPL][decltype(gw_tag)::value], float (&pb)[kTPL][decltype(gw_tag)::value],
                           float (&ta)[decltype(gw_tag)::value], float (&tb)[decltype(gw_tag)::value]) {
    constexpr int GW = decltype(gw_tag)::value;
#pragma unroll
    for (int i = 0; i < kTPL; ++i) {
      const float* bv = (const float*)&sm.io.in.b[q][i * kROW + sl] + h0s;
#pragma unroll
      for (int k = 0; k < GW; ++k) {
        const float a = exp2_hw(dl[i] * a2v[k]);
        const float wu = x[i] * bv[k];
        ar[i][k] = a;
        pa[i][k] = a;
        pb[i][k] = fmaf(a, wu, -wu);  // (abar - 1) u B
      }
    }
#pragma unroll
    for (int i = 1; i < kTPL; ++i) {
#pragma unroll
      for (int k = 0; k < GW; ++k) {
        pb[i][k] = fmaf(pa[i][k], pb[i - 1][k], pb[i][k]);
        pa[i][k] *= pa[i - 1][k];
      }
    }
#pragma unroll
    for (int k = 0; k < GW; ++k) {
      ta[k] = pa[kTPL - 1][k];
      tb[k] = fmaf(ta[k], cinv[k], pb[kTPL - 1][k]);
    }
    row_scan_right(ta, tb);
  };

  const int64_t nck = (L + kTCK - 1) / kTCK;
  // the checkpoint rows of the tile's channels at token t0; element ch * 16 +
  // n of thread (ch, n) is element tid
  auto ckpt_at = [&](int64_t t0) { return p.ckpt + ((b * p.nchunks + t0 / kCkTok) * dim + c0) * kN; };

  // ---- the forward sweep: the state at every chunk start (h units), unless
  // the forward kept it
  if (!p.have_ckpt && nck > 0) {
    tile_load(0, std::false_type());
    bc_load(0, std::false_type());
    for (int64_t ck = 0; ck < nck; ++ck) {
      const int64_t t0 = ck * kTCK;
      tile_store(t0, std::false_type());
      bc_store(t0, std::false_type());
      if (ck + 1 < nck) {
        tile_load(t0 + kTCK, std::false_type());
        bc_load(t0 + kTCK, std::false_type());
      }
      lds_barrier();
      float x[kTPL], dl[kTPL];
      read_xd(x, dl);
#pragma unroll 1
      for (int q = 0; q < kN / 4; ++q) {
        const float4 a24 = kpf[8 * q], ca4 = kpf[8 * q + 1], cin4 = kpf[8 * q + 2];
        const float a2v[4] = {a24.x, a24.y, a24.z, a24.w};
        const float cinv[4] = {cin4.x, cin4.y, cin4.z, cin4.w};
        float ar[kTPL][4], pa[kTPL][4], pb[kTPL][4], ta[4], tb[4];
        forward_pairs(std::integral_constant<int, 4>(), q, 0, x, dl, a2v, cinv, ar, pa, pb, ta, tb);
        // the first lane holds the carry: the checkpoint of this chunk start
        if (sl == 0)
          *(float4*)(ckpt_at(t0) + ch * kN + 4 * q) =
              make_float4(cin4.x * ca4.x, cin4.y * ca4.y, cin4.z * ca4.z, cin4.w * ca4.w);
        // the last lane holds the state after the chunk: the next carry
        if (sl == kLPC - 1) sm.kq[ch][q][0][2] = make_float4(tb[0], tb[1], tb[2], tb[3]);
      }
      lds_barrier();
    }
    // the checkpoints were written by the rows' first lanes and are read by
    // every lane: a barrier that also orders global memory
    __syncthreads();
  }

  // ---- the chunks backwards
  sm.dacc[ch][sl] = 0.0f;  // thread (ch, n); first read after the first chunk's barrier
  const bool want_s = GATE && p.want_dz;
  const int row = lane >> 4;  // the channel's row in the wave
  float hck = 0.0f;           // this thread's (channel, state) checkpoint, a chunk ahead
  if (nck > 0) {
    const int64_t t0 = (nck - 1) * kTCK;
    tile_load(t0, std::true_type());
    bc_load(t0, std::true_type());
    hck = ckpt_at(t0)[tid];
  }
  for (int64_t ck = nck - 1; ck >= 0; --ck) {
    const int64_t t0 = ck * kTCK;
    tile_store(t0, std::true_type());
    bc_store(t0, std::true_type());
    // the state entering the chunk (g units); a chunk wholly in the padding
    // starts from zero (a forward with lengths need not have written it)
    ((float*)&sm.kq[ch][sl >> 2][0][2])[sl & 3] = t0 < Lb ? hck * a_n : 0.0f;
    if (ck > 0) {
      tile_load(t0 - kTCK, std::true_type());
      bc_load(t0 - kTCK, std::true_type());
      hck = ckpt_at(t0 - kTCK)[tid];
    }
    lds_barrier();

    float x[kTPL], dl[kTPL], dsv[kTPL];
    read_xd(x, dl);
    {
      const float4 d4 = *(const float4*)&sm.ds[ch][kTPL * sl];
      dsv[0] = d4.x; dsv[1] = d4.y; dsv[2] = d4.z; dsv[3] = d4.w;
    }
    float ddt[kTPL] = {0.0f, 0.0f, 0.0f, 0.0f}, dxs[kTPL] = {0.0f, 0.0f, 0.0f, 0.0f};
    float svs[kTPL] = {0.0f, 0.0f, 0.0f, 0.0f};
    // the chunk holds the last real token: h_T and the adjoint entering it
    // (dlast, carried unchanged through the padding) give dA's -dlast h_T
    const bool last_real = t0 < Lb && Lb <= t0 + kTCK;

    // one half of a state group (states 2 qh, 2 qh + 1) at a time: a rolled
    // loop keeps one half's values live
#pragma unroll 1
    for (int qh = 0; qh < kN / 2; ++qh) {
      const int q = qh >> 1, hh = qh & 1;
      const float2 a2h = ((const float2*)&kpf[8 * q])[hh], cah = ((const float2*)&kpf[8 * q + 1])[hh];
      const float2 cinh = ((const float2*)&kpf[8 * q + 2])[hh], qinh = ((const float2*)&kpr[8 * q + 3])[hh];
      const float a2v[2] = {a2h.x, a2h.y};
      const float cav[2] = {cah.x, cah.y};
      const float cinv[2] = {cinh.x, cinh.y};
      const float qinv[2] = {qinh.x, qinh.y};

      // 1. the states after each of the lane's tokens (g[i]) and before its
      // first (hin); RA, the product of the lane's abar
      float ar[kTPL][2], g[kTPL][2], hin[2], RA[2];
      {
        float pa[kTPL][2], pb[kTPL][2], ta[2], tb[2];
        forward_pairs(std::integral_constant<int, 2>(), q, 2 * hh, x, dl, a2v, cinv, ar, pa, pb, ta, tb);
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          RA[k] = pa[kTPL - 1][k];
          hin[k] = row_shift1<kRowShr1>(cinv[k], tb[k]);
#pragma unroll
          for (int i = 0; i < kTPL - 1; ++i) g[i][k] = fmaf(pa[i][k], hin[k], pb[i][k]);
          g[kTPL - 1][k] = tb[k];
        }
      }
      // this lane's part of A dA for the chunk; the last lane of the chunk
      // holding the last real token starts it with -dlast h_T
      float dAl[2];
#pragma unroll
      for (int k = 0; k < 2; ++k) dAl[k] = last_real ? -qinv[k] * (g[kTPL - 1][k] * cav[k]) : 0.0f;

      // 2. the adjoint X entering each lane from the right: the lanes' pairs
      // (RA, RB), RB the adjoint leaving the lane for X = 0, scanned right to
      // left from the carry at the last lane
      float X[2];
      {
        float RB[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          float r = 0.0f;
#pragma unroll
          for (int i = kTPL - 1; i >= 0; --i) {
            const float cvk = ((const float*)&sm.io.in.c[q][i * kROW + sl])[2 * hh + k];
            r = i == kTPL - 1 ? dsv[i] * cvk : fmaf(ar[i + 1][k], r, dsv[i] * cvk);
          }
          RB[k] = fmaf(RA[k], qinv[k], ar[0][k] * r);
        }
        row_scan_left(RA, RB);
#pragma unroll
        for (int k = 0; k < 2; ++k) X[k] = row_shift1<kRowShl1>(qinv[k], RB[k]);
        // the row's first lane: the adjoint carried into the chunk before
        if (sl == 0) ((float2*)&sm.kq[ch][q][0][3])[hh] = make_float2(RB[0], RB[1]);
      }

      // 3. the gradients, from the lane's last token down: q_i = ds_i C_i +
      // abar_{i+1} q_{i+1} (X after the last); dB (w u) and dC (ds h) summed
      // over rows r and r + 2, then over tokens i and i + 2 (rows 2k and 2k + 1)
      float qn[2], e[kTPL][2], f[2][2];
#pragma unroll
      for (int i = kTPL - 1; i >= 0; --i) {
        const float2 bv2 = ((const float2*)&sm.io.in.b[q][i * kROW + sl])[hh];
        const float2 cv2 = ((const float2*)&sm.io.in.c[q][i * kROW + sl])[hh];
        const float bv[2] = {bv2.x, bv2.y};
        const float cv[2] = {cv2.x, cv2.y};
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const float dsC = dsv[i] * cv[k];
          const float qq = i == kTPL - 1 ? dsC + X[k] : fmaf(ar[i + 1][k], qn[k], dsC);
          qn[k] = qq;
          const float hp = i == 0 ? hin[k] : g[i - 1][k];
          const float qa = qq * ar[i][k];
          const float m = qa * fmaf(x[i], bv[k], hp);
          ddt[i] += m;
          const float hv = g[i][k] * cav[k];
          if (want_s) svs[i] = fmaf(cv[k], hv, svs[i]);
          dAl[k] = fmaf(-dsC, hv, fmaf(dl[i], m, dAl[k]));
          const float wq = (qa - qq) * cav[k];
          dxs[i] = fmaf(wq, bv[k], dxs[i]);
          e[i][k] = sum_halves(wq * x[i], dsv[i] * hv);
        }
        if (i < 2) {
#pragma unroll
          for (int k = 0; k < 2; ++k) f[i][k] = sum_row_pairs(e[i][k], e[i + 2][k]);
        }
      }
      // A dA: the row's sum (its last lane) added to the chunks before
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        float v = dAl[k];
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xf, 0xf, false));
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x112, 0xf, 0xf, false));
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xf, 0xf, false));
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x118, 0xf, 0xf, false));
        dAl[k] = v;
      }
      if (sl == kLPC - 1) {
        float2* da = (float2*)&sm.dacc[ch][2 * qh];
        const float2 o = *da;
        *da = make_float2(o.x + dAl[0], o.y + dAl[1]);
      }
      // row r of the wave now holds dB (r < 2) or dC (r >= 2) of its lanes'
      // tokens 2 (r & 1) and 2 (r & 1) + 1, summed over the wave's channels
      {
        float* pw = &sm.part[q & 1][w][(row >> 1) * (kTCK * 4) + (kTPL * sl + 2 * (row & 1)) * 4 + 2 * hh];
        *(float2*)pw = make_float2(f[0][0], f[0][1]);
        *(float2*)(pw + 4) = make_float2(f[1][0], f[1][1]);
      }
      if (hh == 0) continue;
      lds_barrier();
      // the block's sum over its waves: two (token, state) entries per
      // thread, waves 0-1 of dB and 2-3 of dC
      {
        const int which = w >> 1, e0 = 2 * (tid & 127);
        const int tok = e0 >> 2, k = e0 & 3;
        const int ei = which * (kTCK * 4) + e0;
        float2 s = *(const float2*)&sm.part[q & 1][0][ei];
#pragma unroll
        for (int v = 1; v < 4; ++v) {
          const float2 o = *(const float2*)&sm.part[q & 1][v][ei];
          s.x += o.x;
          s.y += o.y;
        }
        float* pb0 = p.pbc + (((tile * 2 + which) * p.batch + b) * L + t0) * kN + 4 * q;
        if (t0 + tok < L) *(float2*)(pb0 + tok * kN + k) = s;
      }
    }

    // the chunk's per-(channel, token) sums; every read of `in` ended before
    // the last group's barrier
    *(float4*)&sm.io.out.ddt[ch][kTPL * sl] = make_float4(ddt[0], ddt[1], ddt[2], ddt[3]);
    *(float4*)&sm.io.out.dx[ch][kTPL * sl] = make_float4(dxs[0], dxs[1], dxs[2], dxs[3]);
    if (want_s) *(float4*)&sm.io.out.sv[ch][kTPL * sl] = make_float4(svs[0], svs[1], svs[2], svs[3]);
    lds_barrier();

    // epilogue per (token, 4 channels): d(raw delta), du, dz = dy silu'(z)
    // (C.h + D u), and the sums for d bias
    {
      const int64_t t = t0 + xt;
      if (t < L) {
        const int64_t cb = (row0 + t0) * dim + c0;
        const uint32_t off = xoff(t0);
        float o_dt[4], o_du[4], o_dz[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int cl = 4 * xh + k;
          const float dv = sm.io.out.ddt[cl][xt] * ep_sg[k];
          o_dt[k] = dv;
          o_du[k] = sm.io.out.dx[cl][xt] + ep_dsD[k];
          o_dz[k] = want_s ? fmaf(ep_dyg[k], sm.io.out.sv[cl][xt], ep_dyx[k]) : 0.0f;
          accB[k] += dv;
        }
        store4((IO*)at((const IO*)p.ddelta + cb, off), o_dt);
        store4((IO*)at((const IO*)p.du + cb, off), o_du);
        if (want_s) store4((IO*)at((const IO*)p.dz + cb, off), o_dz);
      }
    }
    lds_barrier();
  }

  // ---- per block: dh0 (the adjoint carried out of the first token), dA
  // (the row's sum over its lanes, plus h0 dh0, times 1/A), dD and d bias
  // partials for this batch entry
  const float dh0v = ((const float*)&sm.kq[ch][sl >> 2][0][3])[sl & 3];
  const int64_t cs0 = (b * dim + c0) * kN;  // the tile's (channel, state) rows; thread (ch, n): + tid
  if (p.dh0) p.dh0[cs0 + tid] = dh0v;
  {
    float dAn = sm.dacc[ch][sl];
    if (p.h0 && Lb > 0) dAn = fmaf(p.h0[cs0 + tid], dh0v, dAn);
    p.pA[cs0 + tid] = dAn * ca_n;
  }
  // dD, d bias: the staging threads' sums over their tokens, then over the
  // 64 token slots of each channel (in LDS, through the dB/dC buffers)
  float* red = &sm.part[0][0][0];  // [2][64][kCPB + 1]
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    red[xt * (kCPB + 1) + 4 * xh + k] = accD[k];
    red[(kTCK + xt) * (kCPB + 1) + 4 * xh + k] = accB[k];
  }
  lds_barrier();
  if (tid < kCPB) {
    float sD = 0.0f, sB = 0.0f;
    for (int j = 0; j < kTCK; ++j) {
      sD += red[j * (kCPB + 1) + tid];
      sB += red[(kTCK + j) * (kCPB + 1) + tid];
    }
    p.pDb[b * dim + c0 + tid] = sD;
    p.pDb[(p.batch + b) * dim + c0 + tid] = sB;
  }
}

template <typename IO, bool GATE>
hipError_t bwd_wave_launch(const BwdArgs& a, hipStream_t stream) {
  const int64_t nblk = a.ntiles * a.batch;
  if (nblk > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((scan_bwd_wave_kernel<IO, GATE>), dim3((unsigned)nblk), dim3(kNT), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_scan_bwd_wave(const BwdArgs& a, bool bf16_io, bool gate, hipStream_t stream) {
  if (a.N != kN || a.dim % kCPB != 0 || a.ntiles * kCPB != a.dim || a.reset ||
      a.nchunks != (a.L + kCkTok - 1) / kCkTok)
    return hipErrorInvalidValue;
  if (bf16_io) return gate ? bwd_wave_launch<bf16_bits, true>(a, stream) : bwd_wave_launch<bf16_bits, false>(a, stream);
  return gate ? bwd_wave_launch<float, true>(a, stream) : bwd_wave_launch<float, false>(a, stream);
}

}  // namespace ssm66
