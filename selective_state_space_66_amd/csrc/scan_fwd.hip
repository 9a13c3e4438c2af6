// scan_fwd.hip -- fused selective scan (forward) for gfx950.
//
// Computes the S6 layer of "Mamba and selective state spaces"
// (zerotofrontier.app/ssm/mamba), section "The selective state-space model":
//   Delta = softplus(raw + bias);  abar = exp(Delta A);
//   h_t = abar h_{t-1} + bbar u_t;  y_t = C_t . h_t + D u_t;  y *= silu(z),
// with bbar from "The discretization the code actually uses" (ZOH, or the
// exponential-Euler rule Delta B), reading the state after writing it.
// Inputs are read once, y is written once and the state never leaves the
// chip -- the fusion argued for in "Why the scan must be fused".
//
// Work decomposition.  A block owns one batch entry and CW consecutive
// channels; its CW x NG threads are (channel, state group) pairs, each group
// holding G of the (padded) NPAD = G NG state entries of its channel in VGPRs
// for the whole sequence.  Tokens run sequentially in chunks of TC:
//   prep      each thread reads u, raw delta and z for TC/NG tokens of its
//             channel, computes Delta and Delta*u (or u) once per (token,
//             channel) and stages them in LDS; D*u and silu(z) stay in its
//             registers for the epilogue.  B and C rows of the chunk are
//             staged in LDS as fp32, interleaved so that one 16-byte read
//             gives a group its B and C for a token.  Raw loads of the next
//             chunk are then issued, to land while the recurrence runs.
//   recurrence (after a barrier) every thread runs its G states over the TC
//             tokens: per update one v_exp_f32 and 4 (Euler) or 6 (ZOH)
//             VALU ops; everything it reads comes from LDS, so waits are
//             in-order and loads pipeline.  It writes one partial readout
//             per token to LDS.
//   epilogue  (after a second barrier) each thread sums the NG partials of
//             its TC/NG tokens, adds D*u, applies the gate and stores y.
// The state carries from chunk to chunk in registers; after the last chunk it
// is written to last_state.
//
// Sequences that do not start from zero or do not fill the batch: h0 (if
// given) is the state before the first token; seq_lens[b] (if given) real
// tokens are followed by padding, which gets Delta = 0 and x = 0 (the state is
// kept) and y = 0; reset[b, t] != 0 (if given) zeroes the state before token
// t.  Resets are block-uniform (a block owns one batch entry), so a chunk
// holding none runs the ordinary batched recurrence.
//
// ZOH fast path: the thread keeps g = A h, for which
//   g_t = abar (g_{t-1} + u B) - u B,
// the exact ZOH update multiplied through by A: no division, no (abar - 1)
// cancellation; the readout uses C / A.  A wave whose channels hold any
// |A| < 1/2 (or A = 0) runs the careful form instead, h-form with
// bbar = Delta B phi(Delta A), phi(k) = (e^k - 1)/k, accurate for every A.
#include <type_traits>

#include "ssm_device.h"
#include "ssm_launch.h"

namespace ssm66 {

namespace {

template <typename IO>
struct RawT;  // register type holding one prefetched io element
template <>
struct RawT<float> { using type = float; };
template <>
struct RawT<bf16_bits> { using type = uint32_t; };

__device__ __forceinline__ float raw_to_f32(float v) { return v; }
__device__ __forceinline__ float raw_to_f32(uint32_t v) { return __uint_as_float(v << 16); }

template <typename IO>
__device__ __forceinline__ typename RawT<IO>::type load_raw(const IO* __restrict__ p) {
  return (typename RawT<IO>::type)(*p);
}

enum class Path { kEuler, kZohFast, kZohCareful };
template <Path P>
using PathTag = std::integral_constant<Path, P>;

// Static shape of one kernel instance.
template <int G_, int NG_>
struct Shape {
  static constexpr int G = G_;                   // states per thread
  static constexpr int NG = NG_;                 // state groups per channel
  static constexpr int NPAD = G * NG;            // padded state count
  static constexpr int CW = 16;                  // channels per block
  static constexpr int THREADS = CW * NG;
  static constexpr int TC = NG == 8 ? 64 : 32;   // tokens per chunk
  static constexpr int RPT = TC / NG;            // tokens each thread prepares and finishes
  static constexpr int BCN = TC * NPAD;          // B (and C) elements per chunk
  static constexpr int BCPT = (BCN + THREADS - 1) / THREADS;
  static constexpr int PSTRIDE = TC * CW + 16;   // partial-readout row stride (bank offset)
  static_assert(TC % NG == 0, "tokens of a chunk must split evenly over the groups");
  static_assert(THREADS % 64 == 0, "whole waves");
  // each thread stages EPT consecutive B (and C) elements of a chunk; with a
  // dense layout (N == NPAD) they are whole groups inside one token
  static constexpr int EPT = BCN / THREADS;
  static_assert(BCN % THREADS == 0 && NPAD % EPT == 0 && EPT % G == 0,
                "a thread stages whole groups of one token");
};

template <class S>
struct Smem {
  float2 dd[S::TC][S::CW];              // (Delta, x): x = Delta*u (Euler) or u (ZOH)
  float bc[S::TC][S::NG][2 * S::G];     // per token and group: G values of B, then of C
  float part[S::NG][S::PSTRIDE];        // partial readouts, [group][token * CW + channel]
  int rst[S::TC];                       // document starts within the chunk (reset flags)
};

// Read 2G consecutive floats (the group's B and C) from LDS.
template <int G>
__device__ __forceinline__ void read_bc(const float* p, float (&b)[G], float (&c)[G]) {
  if constexpr (G == 1) {
    const float2 v = *(const float2*)p;
    b[0] = v.x; c[0] = v.y;
  } else if constexpr (G == 2) {
    const float4 v = *(const float4*)p;
    b[0] = v.x; b[1] = v.y; c[0] = v.z; c[1] = v.w;
  } else {
    static_assert(G == 4, "G is 1, 2 or 4");
    const float4 v0 = *(const float4*)p;
    const float4 v1 = *(const float4*)(p + 4);
    b[0] = v0.x; b[1] = v0.y; b[2] = v0.z; b[3] = v0.w;
    c[0] = v1.x; c[1] = v1.y; c[2] = v1.z; c[3] = v1.w;
  }
}

// One state update for G states at one token; returns the partial readout.
template <int G, Path PATH>
__device__ __forceinline__ float update(float (&st)[G], const float (&Ap)[G], const float (&Aa)[G],
                                        const float (&CA)[G], float2 dd, const float (&Bv)[G],
                                        const float (&Cv)[G]) {
  float acc = 0.0f;
#pragma unroll
  for (int k = 0; k < G; ++k) {
    const float a = exp2_hw(dd.x * Ap[k]);  // abar = exp(Delta A)
    if constexpr (PATH == Path::kEuler) {
      st[k] = fmaf(a, st[k], dd.y * Bv[k]);  // h = abar h + (Delta u) B
      acc = fmaf(Cv[k], st[k], acc);
    } else if constexpr (PATH == Path::kZohFast) {
      const float ub = dd.y * Bv[k];          // u B
      st[k] = fmaf(a, st[k] + ub, -ub);       // g = abar (g + uB) - uB,  g = A h
      acc = fmaf(Cv[k] * CA[k], st[k], acc);  // C h = (C / A) g
    } else {
      const float kap = dd.x * Aa[k];         // Delta A
      const float bbar = dd.x * Bv[k] * zoh_phi(kap, a);
      st[k] = fmaf(a, st[k], bbar * dd.y);    // h = abar h + bbar u
      acc = fmaf(Cv[k], st[k], acc);
    }
  }
  return acc;
}

// The recurrence over the tokens of one chunk for the G states of this thread.
// Full chunks go in batches of U tokens: all LDS reads of a batch are issued
// before its arithmetic, so their latency overlaps, and its U partial readouts
// are written after it.
// CKPT (the training forward): ckpt(t) writes the state before chunk token t
// when t is a multiple of 16 (chunks start at multiples of 16).
template <class S, Path PATH, bool FULL, bool RST = false, bool CKPT = false, class Ckpt>
__device__ __forceinline__ void run_chunk(Smem<S>& sm, float (&st)[S::G], const float (&Ap)[S::G],
                                          const float (&Aa)[S::G], const float (&CA)[S::G],
                                          int nt, int cl, int g, Ckpt&& ckpt) {
  constexpr int G = S::G;
  float* part = &sm.part[g][cl];
  if constexpr (FULL) {
    // batches of U tokens, software-pipelined: the LDS reads of batch j + 1 are
    // issued before the arithmetic of batch j (LDS returns in order, so the
    // waits for batch j do not cover batch j + 1's reads)
    constexpr int U = G >= 4 ? 2 : 4;
    constexpr int NB = S::TC / U;
    static_assert(S::TC % U == 0, "whole batches");
    float2 dd[2][U];
    float Bv[2][U][G], Cv[2][U][G];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      dd[0][j] = sm.dd[j][cl];
      read_bc<G>(&sm.bc[j][g][0], Bv[0][j], Cv[0][j]);
    }
#pragma unroll
    for (int bt = 0; bt < NB; ++bt) {
      const int cur = bt & 1, nxt = cur ^ 1;
      if constexpr (CKPT) {
        if ((bt * U) % 16 == 0) ckpt(bt * U);
      }
      if (bt + 1 < NB) {
#pragma unroll
        for (int j = 0; j < U; ++j) {
          const int t = (bt + 1) * U + j;
          dd[nxt][j] = sm.dd[t][cl];
          read_bc<G>(&sm.bc[t][g][0], Bv[nxt][j], Cv[nxt][j]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      float acc[U];
#pragma unroll
      for (int j = 0; j < U; ++j)
        acc[j] = update<G, PATH>(st, Ap, Aa, CA, dd[cur][j], Bv[cur][j], Cv[cur][j]);
#pragma unroll
      for (int j = 0; j < U; ++j) part[(bt * U + j) * S::CW] = acc[j];
    }
  } else {
    for (int t = 0; t < nt; ++t) {
      if constexpr (CKPT) {
        if (t % 16 == 0) ckpt(t);
      }
      if constexpr (RST) {
        if (sm.rst[t]) {  // a document starts here: forget the state
#pragma unroll
          for (int k = 0; k < G; ++k) st[k] = 0.0f;
        }
      }
      float Bv[G], Cv[G];
      read_bc<G>(&sm.bc[t][g][0], Bv, Cv);
      part[t * S::CW] = update<G, PATH>(st, Ap, Aa, CA, sm.dd[t][cl], Bv, Cv);
    }
  }
}

// Pointers are separate __restrict__ arguments; y must not overlap any input,
// and last_state none but h0 (each thread reads its h0 entries before it
// writes the same entries of last_state).  The host guarantees
// NG * dim < 2^31 (32-bit lane offsets).  CKPT: also write the state before
// every 16th token to ckpt (batch, ceil(L / 16), dim, N), the checkpoints the
// backward pass would otherwise recompute.
template <typename IO, int G, int NG, bool ZOH, bool GATE, bool CKPT>
__global__ __launch_bounds__((Shape<G, NG>::THREADS)) void scan_fwd_kernel(
    const IO* __restrict__ u, const IO* __restrict__ dr, const float* __restrict__ Am,
    const IO* __restrict__ Bm, const IO* __restrict__ Cm, const float* __restrict__ Dm,
    const IO* __restrict__ zz, const float* __restrict__ bias_v, const float* h0,
    const int32_t* __restrict__ seq_lens, const uint8_t* __restrict__ reset,
    IO* __restrict__ y, float* last_state, float* __restrict__ ckpt, const int64_t L,
    const int64_t dim, const int64_t N, const int64_t ntiles, const int softplus) {
  using S = Shape<G, NG>;
  constexpr int CW = S::CW, TC = S::TC, RPT = S::RPT, NPAD = S::NPAD;
  using Raw = typename RawT<IO>::type;

  __shared__ Smem<S> sm;

  // XCD-aware order: consecutive blocks go round-robin to the 8 XCDs, so give
  // each XCD a contiguous run of tiles -- neighbouring tiles share 128-byte
  // lines of u, raw delta, z and y, and then share that XCD's L2.
  const int64_t nblk = (int64_t)gridDim.x;
  const int64_t bid = blockIdx.x;
  const int64_t logical = (nblk % 8 == 0) ? (bid % 8) * (nblk / 8) + bid / 8 : bid;
  const int64_t b = logical / ntiles;
  const int64_t tile = logical - b * ntiles;

  const int tid = threadIdx.x;
  const int cl = tid % CW;  // channel within the tile
  const int g = tid / CW;   // state group
  const int64_t c = tile * CW + cl;
  const bool cvalid = c < dim;
  const bool tile_full = (tile + 1) * CW <= dim;  // block-uniform
  const int64_t cc = cvalid ? c : dim - 1;        // loads of padding lanes stay in bounds
  // offset of (token g, channel cc) from a chunk's first token row; token
  // g + NG i sits i * NG * dim elements further (a uniform step)
  const uint32_t lane_off = (uint32_t)(g * dim + cc);
  const int n0 = g * G;
  const int ngroups = (int)((N + G - 1) / G);  // groups holding real states
  const bool dense_bc = (N == NPAD);           // B, C rows are exactly NPAD wide

  // per-thread channel constants
  float Ap[G], Aa[G], CA[G];
  bool small_a = false;
#pragma unroll
  for (int k = 0; k < G; ++k) {
    const bool real = cvalid && (n0 + k) < N;
    const float a = real ? Am[c * N + n0 + k] : 0.0f;
    Ap[k] = a * kLog2e;
    Aa[k] = a;
    CA[k] = (a != 0.0f) ? 1.0f / a : 0.0f;
    if (real && !(fabsf(a) >= 0.5f)) small_a = true;
  }
  const float bias = (cvalid && bias_v) ? bias_v[c] : 0.0f;
  const float dskip = (cvalid && Dm) ? Dm[c] : 0.0f;
  // a wave with any small |A| runs the careful ZOH form for all its lanes
  const bool careful = ZOH && __any(small_a);

  float st[G];
#pragma unroll
  for (int k = 0; k < G; ++k) {
    float h = 0.0f;
    if (h0 && cvalid && (n0 + k) < N) h = h0[(b * dim + c) * N + n0 + k];
    st[k] = (ZOH && !careful) ? Aa[k] * h : h;  // the fast ZOH path keeps g = A h
  }

  const int64_t nchunks = (L + TC - 1) / TC;
  const int64_t nck = (L + 15) / 16;  // checkpoints per sequence (CKPT)
  const int64_t row0 = b * L;  // first token row of this batch entry
  int64_t Leff = L;            // real tokens of this sequence; the rest is padding
  if (seq_lens) {
    const int64_t sl = seq_lens[b];
    Leff = sl < 0 ? 0 : (sl < L ? sl : L);
  }

  // ---- raw prefetch of one chunk: u, raw delta, z for this thread's tokens,
  // and its share of the chunk's B and C rows (as 32-bit words)
  constexpr int BCW = S::EPT * (int)sizeof(IO) / 4;  // 32-bit words per thread
  Raw ru[RPT], rd[RPT], rz[RPT];
  uint32_t rb[BCW], rc[BCW];
  auto prefetch = [&](int64_t t0) {
    const bool full = t0 + TC <= L;  // uniform
    if (full) {
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const int64_t rowi = (row0 + t0 + NG * i) * dim;  // uniform
        ru[i] = load_raw(u + rowi + lane_off);
        rd[i] = load_raw(dr + rowi + lane_off);
        if constexpr (GATE) rz[i] = load_raw(zz + rowi + lane_off);
      }
    } else {
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        int64_t t = t0 + g + NG * i;
        t = t < L ? t : L - 1;
        const int64_t idx = (row0 + t) * dim + cc;
        ru[i] = load_raw(u + idx);
        rd[i] = load_raw(dr + idx);
        if constexpr (GATE) rz[i] = load_raw(zz + idx);
      }
    }
    // B and C: the chunk's rows are TC * N contiguous elements; words past the
    // last token (or past the tensor) are clamped to its last word
    const int64_t e0 = (row0 + t0) * N;                        // first element
    const int64_t ewords = ((row0 + (full ? t0 + TC : L)) * N * (int64_t)sizeof(IO) + 3) / 4;
    const uint32_t* bw = (const uint32_t*)Bm;
    const uint32_t* cw = (const uint32_t*)Cm;
    const int64_t w0 = e0 * (int64_t)sizeof(IO) / 4;
    if (dense_bc && full) {
#pragma unroll
      for (int i = 0; i < BCW; ++i) {
        rb[i] = bw[w0 + tid * BCW + i];
        rc[i] = cw[w0 + tid * BCW + i];
      }
    } else if (dense_bc) {
#pragma unroll
      for (int i = 0; i < BCW; ++i) {
        int64_t w = w0 + tid * BCW + i;
        w = w < ewords ? w : ewords - 1;
        rb[i] = bw[w];
        rc[i] = cw[w];
      }
    } else {
      // general layout: element by element (dstate below the padded width)
#pragma unroll
      for (int i = 0; i < BCW; ++i) {
        rb[i] = 0u;
        rc[i] = 0u;
      }
#pragma unroll
      for (int i = 0; i < S::EPT; ++i) {
        const int e = tid * S::EPT + i;  // element of the padded chunk
        const int tt = e / NPAD, n = e % NPAD;
        if (e < S::BCN && n < N && t0 + tt < L) {
          const int64_t idx = (row0 + t0 + tt) * N + n;
          uint32_t vb, vc;
          if constexpr (sizeof(IO) == 2) {
            vb = ((const uint16_t*)Bm)[idx];
            vc = ((const uint16_t*)Cm)[idx];
          } else {
            vb = __float_as_uint(((const float*)Bm)[idx]);
            vc = __float_as_uint(((const float*)Cm)[idx]);
          }
          const int sh = (sizeof(IO) == 2) ? 16 * (i & 1) : 0;
          rb[i / (4 / sizeof(IO))] |= vb << sh;
          rc[i / (4 / sizeof(IO))] |= vc << sh;
        }
      }
    }
  };

  // element j (0..NPAD*TC) of the staged B or C word array, as fp32
  auto word_elem = [&](const uint32_t (&w)[BCW], int j) -> float {
    if constexpr (sizeof(IO) == 2)
      return __uint_as_float((j & 1) ? (w[j >> 1] & 0xffff0000u) : (w[j >> 1] << 16));
    else
      return __uint_as_float(w[j]);
  };

  float du[RPT], gz[RPT];
  if (nchunks > 0) prefetch(0);
  for (int64_t ck = 0; ck < nchunks; ++ck) {
    const int64_t t0 = ck * TC;
    const bool full = t0 + TC <= Leff;  // every token of the chunk is real (block-uniform)
    // ---- prep: this thread's tokens of the chunk.  Padding lanes (channel
    // past dim) compute on clamped copies; nothing of theirs is ever stored.
    // Tokens past the sequence (padding, or past L in the last chunk) get
    // Delta = 0 and x = 0, so the state is left as it was after the last real
    // token whatever the padded inputs hold.
    auto prep_token = [&](int i, bool live) {
      const int r = g + NG * i;
      float x = raw_to_f32(ru[i]);
      const float v = raw_to_f32(rd[i]) + bias;
      const float sp = softplus_f(v);
      float dlt = softplus ? sp : v;
      if (!live) {
        dlt = 0.0f;
        x = 0.0f;
      }
      sm.dd[r][cl] = make_float2(dlt, ZOH ? x : dlt * x);
      du[i] = dskip * x;
      gz[i] = 1.0f;
      if constexpr (GATE) gz[i] = silu_f(raw_to_f32(rz[i]));
    };
    if (full) {
#pragma unroll
      for (int i = 0; i < RPT; ++i) prep_token(i, true);
    } else {
#pragma unroll
      for (int i = 0; i < RPT; ++i) prep_token(i, (t0 + g + NG * i) < Leff);
    }
    // ---- stage B and C: this thread's EPT elements are states
    // [ns, ns + EPT) of token tt of the chunk, i.e. whole groups; each group
    // gets its G values of B and then of C.  Tokens past L are zeroed.
    {
      constexpr int EPT = S::EPT;
      const int tt = (tid * EPT) / NPAD;
      const int ns = (tid * EPT) % NPAD;
      const bool live = full || (t0 + tt) < Leff;
#pragma unroll
      for (int q = 0; q < EPT / G; ++q) {
        float* dst = &sm.bc[tt][ns / G + q][0];
#pragma unroll
        for (int k = 0; k < G; ++k) {
          dst[k] = live ? word_elem(rb, q * G + k) : 0.0f;
          dst[G + k] = live ? word_elem(rc, q * G + k) : 0.0f;
        }
      }
    }
    // document starts of this chunk: one flag per token, block-uniform
    bool chunk_resets = false;
    if (reset) {
      int mine = 0;
      if (cl == 0) {
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
          const int r = g + NG * i;
          const int f = (t0 + r < Leff) ? (int)reset[row0 + t0 + r] : 0;
          sm.rst[r] = f;
          mine |= f;
        }
      }
      if (ck + 1 < nchunks) prefetch(t0 + TC);
      chunk_resets = __syncthreads_or(mine) != 0;
    } else {
      if (ck + 1 < nchunks) prefetch(t0 + TC);
      lds_barrier();
    }

    // ---- the recurrence for this thread's states over the chunk's real tokens
    const int64_t nreal = Leff - t0;
    const int nt = (int)(nreal < 0 ? 0 : (nreal < TC ? nreal : TC));
    // the state before chunk token t, in h units, to its checkpoint
    auto write_ckpt = [&](int t) {
      if (cvalid) {
        float* dst = ckpt + ((b * nck + (t0 + t) / 16) * dim + c) * N + n0;
#pragma unroll
        for (int k = 0; k < G; ++k)
          if (n0 + k < N) dst[k] = (ZOH && !careful) ? st[k] * CA[k] : st[k];
      }
    };
    auto run = [&](auto path_tag) {
      constexpr Path PATH = decltype(path_tag)::value;
      if (nt == TC && !chunk_resets)
        run_chunk<S, PATH, true, false, CKPT>(sm, st, Ap, Aa, CA, nt, cl, g, write_ckpt);
      else if (chunk_resets)
        run_chunk<S, PATH, false, true, CKPT>(sm, st, Ap, Aa, CA, nt, cl, g, write_ckpt);
      else
        run_chunk<S, PATH, false, false, CKPT>(sm, st, Ap, Aa, CA, nt, cl, g, write_ckpt);
    };
    if (nt > 0) {
      if constexpr (!ZOH) run(PathTag<Path::kEuler>());
      else if (!careful) run(PathTag<Path::kZohFast>());
      else run(PathTag<Path::kZohCareful>());
    }
    lds_barrier();

    // ---- epilogue: reduce the partial readouts, skip, gate, store
    if (full && tile_full) {
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const int r = g + NG * i;
        float s = sm.part[0][r * CW + cl];
#pragma unroll
        for (int j = 1; j < NG; ++j)
          if (j < ngroups) s += sm.part[j][r * CW + cl];
        store_io(y + (row0 + t0 + NG * i) * dim + lane_off, (s + du[i]) * gz[i]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const int r = g + NG * i;
        const int64_t t = t0 + r;
        if (cvalid && t < L) {
          float out = 0.0f;  // padding outputs 0
          if (t < Leff) {
            float s = sm.part[0][r * CW + cl];
#pragma unroll
            for (int j = 1; j < NG; ++j)
              if (j < ngroups) s += sm.part[j][r * CW + cl];
            out = (s + du[i]) * gz[i];
          }
          store_io(y + (row0 + t) * dim + c, out);
        }
      }
    }
  }

  // ---- final state h_L (the prefill cache)
  if (cvalid && last_state) {
#pragma unroll
    for (int k = 0; k < G; ++k) {
      if (n0 + k < N) {
        const float h = (ZOH && !careful) ? st[k] * CA[k] : st[k];
        last_state[(b * dim + c) * N + n0 + k] = h;
      }
    }
  }
}

template <typename IO, int G, int NG, bool ZOH, bool GATE>
hipError_t launch_one(const ScanParams& p, hipStream_t stream) {
  using S = Shape<G, NG>;
  const int64_t ntiles = (p.dim + S::CW - 1) / S::CW;
  const int64_t nblk = ntiles * p.batch;
  if (nblk > 0x7fffffff) return hipErrorInvalidValue;
  auto kern = p.ckpt ? scan_fwd_kernel<IO, G, NG, ZOH, GATE, true>
                     : scan_fwd_kernel<IO, G, NG, ZOH, GATE, false>;
  hipLaunchKernelGGL(kern, dim3((unsigned)nblk), dim3(S::THREADS), 0, stream, (const IO*)p.u,
                     (const IO*)p.delta, p.A, (const IO*)p.B, (const IO*)p.C, p.D,
                     (const IO*)p.z, p.delta_bias, p.h0, p.seq_lens, p.reset, (IO*)p.y,
                     p.last_state, p.ckpt, p.L, p.dim, p.N, ntiles, p.softplus);
  return hipGetLastError();
}

template <typename IO, int G, int NG>
hipError_t launch_modes(const ScanParams& p, bool zoh, bool gate, hipStream_t stream) {
  if (zoh) return gate ? launch_one<IO, G, NG, true, true>(p, stream) : launch_one<IO, G, NG, true, false>(p, stream);
  return gate ? launch_one<IO, G, NG, false, true>(p, stream) : launch_one<IO, G, NG, false, false>(p, stream);
}

template <typename IO>
hipError_t launch_io(const ScanParams& p, int G, int NG, bool zoh, bool gate, hipStream_t stream) {
  if (G == 4 && NG == 4) return launch_modes<IO, 4, 4>(p, zoh, gate, stream);
  if (G == 2 && NG == 8) return launch_modes<IO, 2, 8>(p, zoh, gate, stream);
  if (G == 1 && NG == 16) return launch_modes<IO, 1, 16>(p, zoh, gate, stream);
  if (G == 2 && NG == 4) return launch_modes<IO, 2, 4>(p, zoh, gate, stream);
  if (G == 1 && NG == 4) return launch_modes<IO, 1, 4>(p, zoh, gate, stream);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_scan_fwd(const ScanParams& p, int io_dtype, int G, int NG, bool zoh, bool gate,
                           hipStream_t stream) {
  if (io_dtype == 1) return launch_io<bf16_bits>(p, G, NG, zoh, gate, stream);
  return launch_io<float>(p, G, NG, zoh, gate, stream);
}

}  // namespace ssm66
