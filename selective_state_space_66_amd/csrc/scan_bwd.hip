// scan_bwd.hip -- backward pass of the fused selective scan for gfx950.
//
// Gradients of the scan in scan_fwd.hip with respect to u, the raw delta, A,
// B, C, D, z, the delta bias and h0, given dy and the gradient of last_state.
// "Mamba and selective state spaces" (zerotofrontier.app/ssm/mamba), "Why the
// scan must be fused": the backward pass stores no states; it reloads the
// inputs, recomputes the states on chip, and runs the reverse recurrence
// (the backward pass of a linear recurrence is a linear recurrence run
// backwards).  With ds_t = dy_t silu(z_t) and the adjoint
//   g_t = ds_t C_t + abar_{t+1} g_{t+1}   (g = dLoss/dh_t),
// the per-update gradients are dabar = g h_{t-1} and dbbar = g u_t, and
// Delta and A are reached through kappa = Delta A (ZOH bbar = Delta B phi(kappa),
// phi(k) = (e^k - 1)/k; exponential-Euler bbar = Delta B).
//
// Decomposition (as the forward): a block owns one batch entry and 16
// channels, its threads are (channel, state group) pairs holding G states.
// Pass 1 runs the states forward through the whole sequence and writes the
// state at every chunk start (TC = 16 tokens) to the workspace.  Pass 2 walks
// the chunks backwards: it recomputes the chunk's states, abar and phi from
// its checkpoint into registers (and the pre-gate output s, for dz), then runs
// the adjoint backwards through the chunk.  Sums over the states of one
// (token, channel) -- dDelta, du, s -- go through LDS across the state groups;
// sums over the channels of one (token, state) -- dB, dC -- go through LDS
// across the block's channels and leave as one partial per channel tile.  A
// second kernel adds the partials (channel tiles for dB, dC; batch entries for
// dA, dD, d bias) in a fixed order: the result does not depend on timing.
//
// Lengths and document starts (the forward of ssm_scan_fwd_ex): tokens at or
// past a sequence's length are staged as Delta = u = dy = 0, so the state and
// the adjoint pass them unchanged (abar = 1, bbar u = 0) and their outputs
// are written as zeros; at a document start the recomputed state restarts
// from zero, the update sees h_{t-1} = 0 and no adjoint is carried to t - 1.
#include <type_traits>

#include "ssm_bwd.h"
#include "ssm_device.h"
#include "ssm_launch.h"

namespace ssm66 {

namespace {

template <int G_, int NG_>
struct BShape {
  static constexpr int G = G_;
  static constexpr int NG = NG_;
  static constexpr int NPAD = G * NG;
  static constexpr int CW = 16;                 // channels per block
  static constexpr int THREADS = CW * NG;
  static constexpr int TC = 16;                 // tokens per chunk (states kept in registers)
  static constexpr int RPT = TC / NG;           // tokens each thread prepares and finishes
  static constexpr int HALF = 8;                // tokens per dB / dC reduction round
  static constexpr int BCN = TC * NPAD;         // B (and C) elements of a chunk
  static constexpr int PST = TC * CW + 16;      // partial row stride
  static_assert(TC % NG == 0 && TC % HALF == 0, "chunk shape");
  static_assert(THREADS % 64 == 0, "whole waves");
};

template <class S>
struct BSmem {
  float4 dd[S::TC][S::CW];                  // (Delta, u, ds, -) per token and channel
  int rst[S::TC];                           // document starts within the chunk
  float bc[S::TC][S::NG][2 * S::G];         // B then C of each group, per token
  float part[3][S::NG][S::PST];             // per-group partial sums per (token, channel)
  float red[2][S::HALF][S::NPAD][S::CW + 1];  // dB, dC contributions per (token, state, channel)
  float chan[2][S::NG][S::CW];              // dD, d bias per (group, channel), at the end
};

// phi(k) = (e^k - 1)/k from a = e^k, and rk = 1/k (from 1/Delta and 1/A:
// a product of two reciprocals instead of one per state).  Below |k| = 1/2:
// 1 + k psi(k), psi a degree-4 polynomial fitted to (phi(k) - 1)/k on
// [-1/2, 1/2] (Chebyshev interpolation; phi within 3e-7 relative in fp32, and
// phi(0) = 1 exactly).  Above: the closed form (a - 1)/k, whose rounding
// error relative to phi is about 2 ulp / |k|.
__device__ __forceinline__ float phi_of(float k, float a, float rk) {
  float p = fmaf(0.0013966609258204699f, k, 0.008395552635192871f);
  p = fmaf(p, k, 0.041666179895401f);
  p = fmaf(p, k, 0.1666627675294876f);
  p = fmaf(p, k, 0.5f);
  p = fmaf(p, k, 1.0f);
  return fabsf(k) < 0.5f ? p : (a - 1.0f) * rk;
}

// phi'(k) given a = e^k, phi = phi(k) and rk = 1/k.  Below |k| = 1/2:
// 1/2 + k chi(k), chi a degree-4 polynomial fitted to (phi'(k) - 1/2)/k on
// [-1/2, 1/2] (within 6e-7 relative in fp32, phi'(0) = 1/2 exactly).  Above:
// the closed form (a - phi)/k.
__device__ __forceinline__ float phi_prime(float k, float a, float phi, float rk) {
  float d = fmaf(0.001197385136038065f, k, 0.006998891942203045f);
  d = fmaf(d, k, 0.03333290293812752f);
  d = fmaf(d, k, 0.1249965950846672f);
  d = fmaf(d, k, 0.3333333432674408f);
  d = fmaf(d, k, 0.5f);
  return fabsf(k) < 0.5f ? d : (a - phi) * rk;
}


// RST: document starts are given (a separate instance, so that the common
// case carries none of their registers).  FAST: the instance for blocks whose
// states all have |A| >= 1/2 (ZOH); with split_fast set, the two instances
// are launched over the same grid and each block runs in the one that fits.
template <typename IO, int G, int NG, bool ZOH, bool GATE, bool RST, bool FAST>
__global__ __launch_bounds__((BShape<G, NG>::THREADS)) void scan_bwd_kernel(const BwdArgs p) {
  using S = BShape<G, NG>;
  constexpr int CW = S::CW, TC = S::TC, RPT = S::RPT, NPAD = S::NPAD, HALF = S::HALF;
  static_assert(ZOH || !FAST, "the fast form is a ZOH form");
  __shared__ BSmem<S> sm;

  const IO* __restrict__ u = (const IO*)p.u;
  const IO* __restrict__ dr = (const IO*)p.delta;
  const IO* __restrict__ Bm = (const IO*)p.B;
  const IO* __restrict__ Cm = (const IO*)p.C;
  const IO* __restrict__ zz = (const IO*)p.z;
  const IO* __restrict__ dyp = (const IO*)p.dy;
  const int64_t L = p.L, dim = p.dim, N = p.N;

  const int64_t nblk = (int64_t)gridDim.x;
  const int64_t bid = blockIdx.x;
  const int64_t logical = (nblk % 8 == 0) ? (bid % 8) * (nblk / 8) + bid / 8 : bid;
  const int64_t b = logical / p.ntiles;
  const int64_t tile = logical - b * p.ntiles;
  const int tid = threadIdx.x;
  const int cl = tid % CW, g = tid / CW;
  const int64_t c = tile * CW + cl;
  const bool cvalid = c < dim;
  const int64_t cc = cvalid ? c : dim - 1;
  const int n0 = g * G;
  const int64_t row0 = b * L;
  int64_t Lb = L;  // real tokens of this sequence; the rest is padding
  if (p.seq_lens) {
    const int64_t sl = p.seq_lens[b];
    Lb = sl < 0 ? 0 : (sl < L ? sl : L);
  }

  float Aa[G], Ap[G], CA[G];
  bool small_a = false;
#pragma unroll
  for (int k = 0; k < G; ++k) {
    const bool real = cvalid && (n0 + k) < N;
    Aa[k] = real ? p.A[c * N + n0 + k] : 0.0f;
    Ap[k] = Aa[k] * kLog2e;
    CA[k] = Aa[k] != 0.0f ? 1.0f / Aa[k] : 0.0f;
    if (real && !(fabsf(Aa[k]) >= 0.5f)) small_a = true;
  }
  // pass 2 takes the g form (g = A h) in the FAST instance: every state of
  // the block has |A| >= 1/2, where abar - 1 and 1/A are accurate enough
  // (block-uniform choice; the other blocks leave)
  if (p.split_fast) {
    const bool block_fast = ZOH && !__syncthreads_or(small_a);
    if (block_fast != FAST) return;
  }
  // pass 1 under ZOH keeps g = A h, as the forward's fast form, unless a lane
  // of the wave has a small |A| (wave-uniform choice)
  const bool fast = FAST || (ZOH && !__any(small_a));
  const float bias = p.bias ? p.bias[cc] : 0.0f;
  const float dskip = p.D ? p.D[cc] : 0.0f;

  // ---- raw inputs of one chunk, read into registers a chunk ahead through
  // addresses clamped into the tensors (no branch around a load): u, raw
  // Delta (and dy, z in pass 2) of this thread's tokens, and the B (and C)
  // values of one (token, state group) -- TC * NG of them, one per thread.
  static_assert(TC * NG == S::THREADS, "one (token, group) of B and C per thread");
  const int btt = tid / NG, bgg = tid % NG;
  IO ru[RPT], rdl[RPT], rdy[RPT], rz[RPT], rb[G], rc[G];
  int rrs[RPT];
  auto load_raw = [&](int64_t t0, bool bwd) {
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int64_t t = t0 + g + NG * i;
      const int64_t tr = t < L ? t : L - 1;
      const int64_t idx = (row0 + tr) * dim + cc;
      ru[i] = u[idx];
      rdl[i] = dr[idx];
      if constexpr (RST) rrs[i] = (int)p.reset[row0 + tr];
      if (bwd) {
        rdy[i] = dyp[idx];
        if constexpr (GATE) rz[i] = zz[idx];
      }
    }
    const int64_t t = t0 + btt;
    const int64_t base = (row0 + (t < L ? t : L - 1)) * N;
#pragma unroll
    for (int k = 0; k < G; ++k) {
      const int n = bgg * G + k;
      const int64_t bi = base + (n < N ? n : N - 1);
      rb[k] = Bm[bi];
      if (bwd) rc[k] = Cm[bi];
    }
  };

  // ---- stage one chunk from the raw registers: (Delta, u, ds) per (token,
  // channel), B and C per (token, state); the epilogue values of this
  // thread's tokens stay in registers.  Tokens past L get zeros, and so do u
  // and dy of channels past dim.
  float e_dy[RPT], e_sv[RPT], e_dg[RPT], e_u[RPT], e_ds[RPT];
  // returns whether this thread staged a document start (cl == 0 threads
  // stage the chunk's flags)
  auto stage = [&](int64_t t0, bool bwd) -> int {
    int starts = 0;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = g + NG * i;
      const bool live = t0 + r < Lb;
      if constexpr (RST) {
        if (cl == 0) {
          const int f = (live && rrs[i] != 0) ? 1 : 0;
          sm.rst[r] = f;
          starts |= f;
        }
      }
      const float x = (live && cvalid) ? to_f32(ru[i]) : 0.0f;
      const float v = to_f32(rdl[i]) + bias;
      const float dl = live ? (p.softplus ? softplus_f(v) : v) : 0.0f;
      float ds = 0.0f;
      if (bwd) {
        const float dyv = (live && cvalid) ? to_f32(rdy[i]) : 0.0f;
        float gz = 1.0f, dg = 0.0f;
        if constexpr (GATE) {
          const float zv = to_f32(rz[i]);
          const float sg = rcp_hw(1.0f + exp2_hw(-zv * kLog2e));  // sigma(z)
          gz = zv * sg;                                          // silu(z)
          dg = sg * fmaf(zv, 1.0f - sg, 1.0f);                   // silu'(z)
        }
        ds = dyv * gz;
        e_dy[i] = dyv;
        e_dg[i] = dg;
        e_u[i] = x;
        e_ds[i] = ds;
        // d softplus / dv = sigma(v)
        e_sv[i] = p.softplus ? rcp_hw(1.0f + exp2_hw(-v * kLog2e)) : 1.0f;
      }
      // 1/Delta for the closed forms of phi and phi' (unused where Delta = 0:
      // the polynomial branch is taken there)
      sm.dd[r][cl] = make_float4(dl, x, ds, rcp_hw(dl));
    }
    const bool live = t0 + btt < Lb;
#pragma unroll
    for (int k = 0; k < G; ++k) {
      const bool ok = live && bgg * G + k < N;
      sm.bc[btt][bgg][k] = ok ? to_f32(rb[k]) : 0.0f;
      if (bwd) sm.bc[btt][bgg][G + k] = ok ? to_f32(rc[k]) : 0.0f;
    }
    return starts;
  };
  // the barrier after staging; with document starts it also tells every
  // thread whether the chunk has one (block-uniform)
  auto staged = [&](int starts) -> bool {
    if constexpr (RST) return __syncthreads_or(starts) != 0;
    lds_barrier();
    return false;
  };

  auto update_state = [&](float& h, float a, float bw, float dl, float x, float Bv) {
    // h = abar h + bbar u, bbar = Delta B phi (ZOH; bw = phi) or Delta B (Euler)
    h = fmaf(a, h, (ZOH ? dl * bw : dl) * Bv * x);
  };

  // ---- pass 1: the states forward, one checkpoint per chunk start.  Under
  // ZOH's fast form h holds g = A h: g = abar (g + u B) - u B exactly, and the
  // checkpoint is g / A.
  float h[G];
#pragma unroll
  for (int k = 0; k < G; ++k) {
    h[k] = (p.h0 && cvalid && n0 + k < N) ? p.h0[(b * dim + c) * N + n0 + k] : 0.0f;
    if (fast) h[k] *= Aa[k];
  }
  auto p1_tokens = [&](auto full_tag, auto fast_tag, int nt) {
    constexpr bool FULL = decltype(full_tag)::value, P1F = decltype(fast_tag)::value;
#pragma unroll
    for (int t = 0; t < TC; ++t) {
      if (FULL || t < nt) {
        if (RST && !FULL && sm.rst[t]) {  // a document starts here: forget the state
#pragma unroll
          for (int k = 0; k < G; ++k) h[k] = 0.0f;
        }
        const float4 d4 = sm.dd[t][cl];
#pragma unroll
        for (int k = 0; k < G; ++k) {
          const float Bv = sm.bc[t][g][k];
          const float a = exp2_hw(d4.x * Ap[k]);
          if constexpr (P1F) {
            const float ub = d4.y * Bv;
            h[k] = fmaf(a, h[k] + ub, -ub);
          } else {
            const float phi = ZOH ? phi_of(d4.x * Aa[k], a, d4.w * CA[k]) : 1.0f;
            update_state(h[k], a, phi, d4.x, d4.y, Bv);
          }
        }
      }
    }
  };
  const int64_t p1_chunks = p.have_ckpt ? 0 : p.nchunks;
  if (p1_chunks > 0) load_raw(0, false);
  for (int64_t ck = 0; ck < p1_chunks; ++ck) {
    const int64_t t0 = ck * TC;
    if (cvalid) {
#pragma unroll
      for (int k = 0; k < G; ++k)
        if (n0 + k < N)
          p.ckpt[((b * p.nchunks + ck) * dim + c) * N + n0 + k] = fast ? h[k] * CA[k] : h[k];
    }
    const int starts = stage(t0, false);
    if (ck + 1 < p.nchunks) load_raw(t0 + TC, false);
    const bool rst = staged(starts);
    const int nt = (int)(L - t0 < TC ? L - t0 : TC);
    if (nt == TC && !rst) {
      if (fast) p1_tokens(std::true_type(), std::true_type(), nt);
      else p1_tokens(std::true_type(), std::false_type(), nt);
    } else {
      if (fast) p1_tokens(std::false_type(), std::true_type(), nt);
      else p1_tokens(std::false_type(), std::false_type(), nt);
    }
    lds_barrier();
  }

  // ---- pass 2: the chunks backwards
  float gad[G], dA[G];
#pragma unroll
  for (int k = 0; k < G; ++k) {
    gad[k] = (p.dlast && cvalid && n0 + k < N) ? p.dlast[(b * dim + c) * N + n0 + k] : 0.0f;
    dA[k] = 0.0f;
  }
  float accD = 0.0f, accB = 0.0f;  // this thread's tokens: sum ds u, sum d(raw delta)
  // the chunk's checkpoint is read with its inputs, a chunk ahead
  float hnext[G];
  auto load_ckpt = [&](int64_t ck) {
#pragma unroll
    for (int k = 0; k < G; ++k)
      hnext[k] = p.ckpt[((b * p.nchunks + ck) * dim + cc) * N + (n0 + k < N ? n0 + k : N - 1)];
  };
  if (p.nchunks > 0) {
    load_raw((p.nchunks - 1) * TC, true);
    load_ckpt(p.nchunks - 1);
  }
  for (int64_t ck = p.nchunks - 1; ck >= 0; --ck) {
    const int64_t t0 = ck * TC;
    const int nt = (int)(L - t0 < TC ? L - t0 : TC);
    const int starts = stage(t0, true);
    // a chunk wholly in the padding starts from zero (a forward with lengths
    // need not have written its checkpoint); its tokens change nothing
    float hst[G];
#pragma unroll
    for (int k = 0; k < G; ++k) hst[k] = (cvalid && n0 + k < N && t0 < Lb) ? hnext[k] : 0.0f;
    if (ck > 0) {
      load_raw(t0 - TC, true);
      load_ckpt(ck - 1);
    }
    const bool rst = staged(starts);

    // recompute: the chunk's states and abar (and phi, off the fast form).
    // On the fast form the registers hold g = A h; gst is the chunk start's.
    float hs[TC][G], as[TC][G], ps[TC][G], gst[G];
#pragma unroll
    for (int k = 0; k < G; ++k) {
      gst[k] = FAST ? hst[k] * Aa[k] : hst[k];
      h[k] = gst[k];
    }
    const bool want_s = GATE && p.want_dz;
    // off the fast form the partial pre-gate readout s (for dz) is taken here
    auto recompute = [&](auto full_tag) {
      constexpr bool FULL = decltype(full_tag)::value;
#pragma unroll
      for (int t = 0; t < TC; ++t) {
        if (FULL || t < nt) {
          if (RST && !FULL && sm.rst[t]) {
#pragma unroll
            for (int k = 0; k < G; ++k) h[k] = 0.0f;
          }
          const float4 d4 = sm.dd[t][cl];
          float acc = 0.0f;
#pragma unroll
          for (int k = 0; k < G; ++k) {
            const float Bv = sm.bc[t][g][k];
            const float a = exp2_hw(d4.x * Ap[k]);
            if constexpr (FAST) {
              const float ub = d4.y * Bv;
              h[k] = fmaf(a, h[k] + ub, -ub);
            } else {
              const float phi = ZOH ? phi_of(d4.x * Aa[k], a, d4.w * CA[k]) : 1.0f;
              update_state(h[k], a, phi, d4.x, d4.y, Bv);
              ps[t][k] = phi;
              acc = fmaf(sm.bc[t][g][G + k], h[k], acc);
            }
            hs[t][k] = h[k];
            as[t][k] = a;
          }
          if (!FAST && want_s) sm.part[0][g][t * CW + cl] = acc;
        }
      }
    };
    const bool full = nt == TC && !rst;
    if (full) recompute(std::true_type());
    else recompute(std::false_type());
    if constexpr (FAST) {
      // the final state h_T (the state after the last real token: padding
      // tokens leave it unchanged) enters dA on the fast form
      if (t0 < Lb && Lb <= t0 + TC) {
#pragma unroll
        for (int k = 0; k < G; ++k) dA[k] = fmaf(-gad[k], h[k] * CA[k], dA[k]);
      }
    } else {
      lds_barrier();
      // dz = dy s silu'(z), s = C.h + D u (this thread's tokens)
      if constexpr (GATE) {
        if (p.want_dz) {
#pragma unroll
          for (int i = 0; i < RPT; ++i) {
            const int r = g + NG * i;
            const int64_t t = t0 + r;
            if (cvalid && r < nt) {
              float sv = fmaf(dskip, e_u[i], 0.0f);
              for (int j = 0; j < NG; ++j) sv += sm.part[0][j][r * CW + cl];
              store_io((IO*)p.dz + (row0 + t) * dim + c, e_dy[i] * sv * e_dg[i]);
            }
          }
        }
      }
      lds_barrier();
    }

    // the adjoint backwards through the chunk, in two rounds of HALF tokens
#pragma unroll
    for (int half = TC / HALF - 1; half >= 0; --half) {
      auto reverse = [&](auto full_tag) {
        constexpr bool FULL = decltype(full_tag)::value;
#pragma unroll
        for (int tt = HALF - 1; tt >= 0; --tt) {
          const int t = half * HALF + tt;
          if (FULL || t < nt) {
            const float4 d4 = sm.dd[t][cl];
            const float dl = d4.x, x = d4.y, ds = d4.z, rdl = d4.w;
            const float xdl = x * dl;
            // a document start: the update saw h_{t-1} = 0 and carries nothing back
            const bool start = RST && !FULL && sm.rst[t] != 0;
            float ddt = 0.0f, dx = 0.0f, sacc = 0.0f;
#pragma unroll
            for (int k = 0; k < G; ++k) {
              const float Bv = sm.bc[t][g][k], Cv = sm.bc[t][g][G + k];
              const float a = as[t][k];
              const float hp = start ? 0.0f : (t > 0 ? hs[t > 0 ? t - 1 : 0][k] : gst[k]);
              // q is the adjoint of h_t (q abar carries it to t - 1); the
              // adjoints of abar and bbar u are q h_{t-1} and q.  Channels
              // past dim stage u = ds = 0, so their dB, dC terms are zero.
              const float q = fmaf(ds, Cv, gad[k]);
              const float qa = q * a;
              if constexpr (FAST) {
                // g form (hp, hs hold g = A h; bbar u = (abar - 1) u B / A):
                // dDelta: q abar (g_{t-1} + u B); dB, du: w u, w B with
                // w = q (abar - 1) / A; dA collects Delta q abar (g_{t-1} +
                // u B) - ds C h here (times 1/A at the end)
                const float hv = hs[t][k] * CA[k];
                const float Ch = Cv * hv;
                if (want_s) sacc += Ch;
                const float m = qa * fmaf(x, Bv, hp);
                ddt += m;
                dA[k] = fmaf(-ds, Ch, fmaf(dl, m, dA[k]));
                const float w = (qa - q) * CA[k];
                sm.red[0][tt][n0 + k][cl] = w * x;
                sm.red[1][tt][n0 + k][cl] = ds * hv;
                dx = fmaf(w, Bv, dx);
              } else {
                const float xB = x * Bv;
                if constexpr (ZOH) {
                  const float phi = ps[t][k];
                  const float dphi = phi_prime(dl * Aa[k], a, phi, rdl * CA[k]);
                  // dDelta: q (h_{t-1} A + u B) abar (d bbar/dDelta = abar B);
                  // dA: q (h_{t-1} Delta abar + u B Delta^2 phi'); dB: q u Delta
                  // phi; du: q Delta B phi
                  ddt = fmaf(qa, fmaf(hp, Aa[k], xB), ddt);
                  dA[k] = fmaf(dl, fmaf(q * xB * dl, dphi, qa * hp), dA[k]);
                  const float qp = q * phi;
                  sm.red[0][tt][n0 + k][cl] = qp * xdl;
                  dx = fmaf(qp, dl * Bv, dx);
                } else {
                  ddt = fmaf(qa * hp, Aa[k], fmaf(q, xB, ddt));
                  dA[k] = fmaf(qa * hp, dl, dA[k]);
                  sm.red[0][tt][n0 + k][cl] = q * xdl;
                  dx = fmaf(q * dl, Bv, dx);
                }
                sm.red[1][tt][n0 + k][cl] = ds * hs[t][k];
              }
              gad[k] = start ? 0.0f : qa;
            }
            sm.part[0][g][t * CW + cl] = ddt;
            sm.part[1][g][t * CW + cl] = dx;
            if (FAST && want_s) sm.part[2][g][t * CW + cl] = sacc;
          }
        }
      };
      if (full) reverse(std::true_type());
      else reverse(std::false_type());
      lds_barrier();
      // dB, dC of these HALF tokens: sum over the block's channels
      for (int e = tid; e < 2 * HALF * NPAD; e += S::THREADS) {
        const int which = e / (HALF * NPAD);
        const int rem = e - which * HALF * NPAD;
        const int tt = rem / NPAD, n = rem % NPAD;
        const int t = half * HALF + tt;
        if (t < nt && n < N) {
          float s = 0.0f;
#pragma unroll
          for (int q = 0; q < CW; ++q) s += sm.red[which][tt][n][q];
          p.pbc[(((tile * 2 + which) * p.batch + b) * L + t0 + t) * N + n] = s;
        }
      }
      lds_barrier();
    }

    // epilogue: d(raw delta), du (and on the fast form dz = dy s silu'(z),
    // s = C.h + D u); sums for dD and d bias
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = g + NG * i;
      const int64_t t = t0 + r;
      if (r < nt) {
        float ddt = 0.0f, dx = e_ds[i] * dskip, sv = dskip * e_u[i];
        for (int j = 0; j < NG; ++j) {
          ddt += sm.part[0][j][r * CW + cl];
          dx += sm.part[1][j][r * CW + cl];
          if (FAST && want_s) sv += sm.part[2][j][r * CW + cl];
        }
        const float dv = t < Lb ? ddt * e_sv[i] : 0.0f;  // padding: no step size
        accB += dv;
        accD = fmaf(e_ds[i], e_u[i], accD);
        if (cvalid) {
          store_io((IO*)p.ddelta + (row0 + t) * dim + c, dv);
          store_io((IO*)p.du + (row0 + t) * dim + c, dx);
          if constexpr (GATE && FAST) {
            if (want_s) store_io((IO*)p.dz + (row0 + t) * dim + c, e_dy[i] * sv * e_dg[i]);
          }
        }
      }
    }
    lds_barrier();
  }

  // ---- per-block results: dh0 (the carried adjoint is abar_0 g_0), dA,
  // dD and d bias partials for this batch entry.  On the fast form dA holds
  // A dA - h0 dh0 (the sum over the updates of q dbbar/dA u, which it lacks,
  // equals sum ds C h + dlast h_T - h0 dh0: the adjoint identity of a linear
  // recurrence); with no real token there is nothing to add.
  if (cvalid) {
#pragma unroll
    for (int k = 0; k < G; ++k) {
      if (n0 + k < N) {
        float dAk = dA[k];
        if constexpr (FAST) {
          if (p.h0 && Lb > 0) dAk = fmaf(p.h0[(b * dim + c) * N + n0 + k], gad[k], dAk);
          dAk *= CA[k];
        }
        if (p.dh0) p.dh0[(b * dim + c) * N + n0 + k] = gad[k];
        p.pA[(b * dim + c) * N + n0 + k] = dAk;
      }
    }
  }
  sm.chan[0][g][cl] = accD;
  sm.chan[1][g][cl] = accB;
  lds_barrier();
  if (g == 0 && cvalid) {
    float sD = 0.0f, sB = 0.0f;
    for (int j = 0; j < NG; ++j) {
      sD += sm.chan[0][j][cl];
      sB += sm.chan[1][j][cl];
    }
    p.pDb[b * dim + c] = sD;
    p.pDb[(p.batch + b) * dim + c] = sB;
  }
}

// dB, dC: add the channel tiles' partials in tile order, round to the io dtype.
// A thread takes four consecutive elements (16-byte reads; n is a multiple of
// 4 when every row of B holds a multiple of 4 states, else one element).
template <typename IO, int V>
__global__ __launch_bounds__(256) void bwd_finalize_bc(const float* __restrict__ pbc,
                                                       IO* __restrict__ dB, IO* __restrict__ dC,
                                                       const int64_t ntiles, const int64_t n) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * V;
  if (i >= n) return;
  float sb[V], sc[V];
#pragma unroll
  for (int k = 0; k < V; ++k) sb[k] = sc[k] = 0.0f;
#pragma unroll 4
  for (int64_t tl = 0; tl < ntiles; ++tl) {
    const float* pb = pbc + (tl * 2) * n + i;
    const float* pc = pb + n;
    if constexpr (V == 4) {
      const float4 b4 = *(const float4*)pb, c4 = *(const float4*)pc;
      sb[0] += b4.x; sb[1] += b4.y; sb[2] += b4.z; sb[3] += b4.w;
      sc[0] += c4.x; sc[1] += c4.y; sc[2] += c4.z; sc[3] += c4.w;
    } else {
      sb[0] += pb[0];
      sc[0] += pc[0];
    }
  }
#pragma unroll
  for (int k = 0; k < V; ++k) {
    store_io(dB + i + k, sb[k]);
    store_io(dC + i + k, sc[k]);
  }
}

// dA (dim * N), dD and d bias (dim): add the batch entries' partials in order.
__global__ __launch_bounds__(256) void bwd_finalize_params(
    const float* __restrict__ pA, const float* __restrict__ pDb, float* __restrict__ dA,
    float* __restrict__ dD, float* __restrict__ dbias, const int64_t batch, const int64_t dim,
    const int64_t N) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < dim * N) {
    float s = 0.0f;
    for (int64_t b = 0; b < batch; ++b) s += pA[b * dim * N + i];
    dA[i] = s;
  }
  if (i < dim) {
    float sD = 0.0f, sB = 0.0f;
    for (int64_t b = 0; b < batch; ++b) {
      sD += pDb[b * dim + i];
      sB += pDb[(batch + b) * dim + i];
    }
    if (dD) dD[i] = sD;
    if (dbias) dbias[i] = sB;
  }
}

template <typename IO, int G, int NG, bool ZOH, bool GATE, bool FAST>
hipError_t bwd_launch_rst(const BwdArgs& a, hipStream_t stream) {
  using S = BShape<G, NG>;
  const int64_t nblk = a.ntiles * a.batch;
  if (a.reset)
    hipLaunchKernelGGL((scan_bwd_kernel<IO, G, NG, ZOH, GATE, true, FAST>), dim3((unsigned)nblk),
                       dim3(S::THREADS), 0, stream, a);
  else
    hipLaunchKernelGGL((scan_bwd_kernel<IO, G, NG, ZOH, GATE, false, FAST>), dim3((unsigned)nblk),
                       dim3(S::THREADS), 0, stream, a);
  return hipGetLastError();
}

// ZOH with N > 8 launches the exact instance and the fast one over the same
// grid; each block runs in one of them.  Other shapes and Euler run the exact
// instance alone.
template <typename IO, int G, int NG, bool ZOH, bool GATE>
hipError_t bwd_launch_one(BwdArgs a, hipStream_t stream) {
  if (a.ntiles * a.batch > 0x7fffffff) return hipErrorInvalidValue;
  constexpr bool kSplit = ZOH && G == 2 && NG == 8;
  a.split_fast = kSplit ? 1 : 0;
  const hipError_t e = bwd_launch_rst<IO, G, NG, ZOH, GATE, false>(a, stream);
  if (e != hipSuccess || !kSplit) return e;
  return bwd_launch_rst<IO, G, NG, ZOH, GATE, kSplit>(a, stream);
}

template <typename IO, int G, int NG>
hipError_t bwd_modes(const BwdArgs& a, bool zoh, bool gate, hipStream_t stream) {
  if (zoh) return gate ? bwd_launch_one<IO, G, NG, true, true>(a, stream)
                       : bwd_launch_one<IO, G, NG, true, false>(a, stream);
  return gate ? bwd_launch_one<IO, G, NG, false, true>(a, stream)
              : bwd_launch_one<IO, G, NG, false, false>(a, stream);
}

template <typename IO>
hipError_t bwd_io(const ScanBwdParams& q, bool zoh, bool gate, hipStream_t stream) {
  BwdArgs a;
  a.u = q.u; a.delta = q.delta; a.B = q.B; a.C = q.C; a.z = q.z; a.dy = q.dy;
  a.A = q.A; a.D = q.D; a.bias = q.delta_bias; a.h0 = q.h0; a.dlast = q.dlast;
  a.seq_lens = q.seq_lens; a.reset = q.reset;
  a.du = q.du; a.ddelta = q.ddelta; a.dz = q.dz; a.dh0 = q.dh0;
  a.batch = q.batch; a.L = q.L; a.dim = q.dim; a.N = q.N;
  a.ntiles = (q.dim + 15) / 16;
  a.nchunks = (q.L + 15) / 16;
  a.softplus = q.softplus;
  a.want_dz = q.dz != nullptr;
  // workspace: checkpoints, dB/dC partials, dA partials, dD/dbias partials
  char* w = (char*)q.workspace;
  a.ckpt = q.ckpt ? (float*)q.ckpt : (float*)w;
  a.have_ckpt = q.ckpt != nullptr;
  w += scan_bwd_ckpt_bytes(q.batch, q.L, q.dim, q.N);
  a.pbc = (float*)w;
  w += (size_t)a.ntiles * 2 * q.batch * q.L * q.N * sizeof(float);
  a.pA = (float*)w;
  w += (size_t)q.batch * q.dim * q.N * sizeof(float);
  a.pDb = (float*)w;
  hipError_t e;
  // ZOH, N = 16, no document starts, aligned rows: the fast tiles go to the
  // time-parallel kernel, the others to this file's exact instance
  auto al16 = [](const void* ptr) { return ptr == nullptr || (uintptr_t)ptr % 16 == 0; };
  const bool wave = zoh && q.N == 16 && !q.reset && q.dim % 16 == 0 && al16(q.u) && al16(q.delta) &&
                    al16(q.z) && al16(q.dy) && al16(q.du) && al16(q.ddelta) && al16(q.dz) && al16(q.B) &&
                    al16(q.C);
  if (wave) {
    a.split_fast = 1;
    e = gate ? bwd_launch_rst<IO, 2, 8, true, true, false>(a, stream)
             : bwd_launch_rst<IO, 2, 8, true, false, false>(a, stream);
    if (e == hipSuccess) e = launch_scan_bwd_wave(a, sizeof(IO) == 2, gate, stream);
  } else if (q.N <= 4) e = bwd_modes<IO, 1, 4>(a, zoh, gate, stream);
  else if (q.N <= 8) e = bwd_modes<IO, 2, 4>(a, zoh, gate, stream);
  else e = bwd_modes<IO, 2, 8>(a, zoh, gate, stream);
  if (e != hipSuccess) return e;
  const int64_t nbc = q.batch * q.L * q.N;
  if (nbc > 0) {
    // the partials are 256-byte aligned sections; 4 elements per thread
    // where n (and so each section's offset in elements) is a multiple of 4
    if (nbc % 4 == 0)
      hipLaunchKernelGGL((bwd_finalize_bc<IO, 4>), dim3((unsigned)((nbc / 4 + 255) / 256)), dim3(256), 0,
                         stream, a.pbc, (IO*)q.dB, (IO*)q.dC, a.ntiles, nbc);
    else
      hipLaunchKernelGGL((bwd_finalize_bc<IO, 1>), dim3((unsigned)((nbc + 255) / 256)), dim3(256), 0,
                         stream, a.pbc, (IO*)q.dB, (IO*)q.dC, a.ntiles, nbc);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t np = q.dim * q.N;
  hipLaunchKernelGGL(bwd_finalize_params, dim3((unsigned)((np + 255) / 256)), dim3(256), 0, stream,
                     a.pA, a.pDb, q.dA, q.dD, q.ddelta_bias, q.batch, q.dim, q.N);
  return hipGetLastError();
}

}  // namespace

size_t scan_bwd_ckpt_bytes(int64_t batch, int64_t L, int64_t dim, int64_t N) {
  // 256-byte aligned sections
  const size_t raw = (size_t)batch * ((L + 15) / 16) * dim * N * sizeof(float);
  return (raw + 255) / 256 * 256;
}

size_t scan_bwd_workspace_bytes(int64_t batch, int64_t L, int64_t dim, int64_t N) {
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t ntiles = (size_t)((dim + 15) / 16);
  return scan_bwd_ckpt_bytes(batch, L, dim, N) + al(ntiles * 2 * batch * L * N * sizeof(float)) +
         al((size_t)batch * dim * N * sizeof(float)) + al((size_t)2 * batch * dim * sizeof(float));
}

hipError_t launch_scan_bwd(const ScanBwdParams& q, int io_dtype, bool zoh, bool gate,
                           hipStream_t stream) {
  if (io_dtype == 1) return bwd_io<bf16_bits>(q, zoh, gate, stream);
  return bwd_io<float>(q, zoh, gate, stream);
}

}  // namespace ssm66
