// ssm_api.hip -- the C ABI declared in include/ssm66.h.
//
// Argument validation runs before any HIP call, so an invalid call returns its
// status without touching a device and with nothing enqueued.  A valid call
// chooses a kernel instance and enqueues one launch on the caller's stream.
#include <stdint.h>
#include <stdlib.h>

#include "../../include/ssm66.h"
#include "ssm_launch.h"

namespace {

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// a * b * c without int64 overflow; false on overflow
bool mul3(int64_t a, int64_t b, int64_t c, int64_t* out) {
  __int128 r = (__int128)a * b * c;
  if (r > INT64_MAX) return false;
  *out = (int64_t)r;
  return true;
}

int check_common(int64_t batch, int64_t len, int64_t dim, int64_t dstate, int io_dtype,
                 int softplus, int dt_mode) {
  if (batch < 0 || len < 0 || dim < 0) return SSM_ERR_SHAPE;
  if (dstate < 1 || dstate > 16) return SSM_ERR_SHAPE;
  if (io_dtype != SSM_F32 && io_dtype != SSM_BF16) return SSM_ERR_DTYPE;
  if (softplus != 0 && softplus != 1) return SSM_ERR_FLAG;
  if (dt_mode != SSM_DT_ZOH && dt_mode != SSM_DT_EULER) return SSM_ERR_FLAG;
  int64_t tmp;
  if (!mul3(batch, len, dim, &tmp) || !mul3(batch, len, dstate, &tmp) ||
      !mul3(batch, dim, dstate, &tmp) || !mul3(dim, dstate, 4, &tmp))
    return SSM_ERR_SHAPE;
  return SSM_OK;
}

// Kernel choice, from sweeps on MI355X (bf16, N 16, ZOH, gate):
// - fewer than 1024 (batch x channel) rows and at least 128 tokens: the
//   time-parallel kernel with four waves per row (88 against 153 us for one
//   wave per row at 1 x 8192 x 256; slower from 1024 rows: 56 against 43 us
//   at 1 x 2048 x 1024);
// - sequences under 256 tokens: the sequential kernel (19 against 30 us at
//   8 x 64 x 1536; 37 against 31 us at 8 x 256 x 1536);
// - 32768 rows or more: the sequential kernel with 4 states per lane, whose
//   2048 waves fill every SIMD twice (426 against 484 us at 8 x 2048 x 4096);
// - everything between: the time-parallel kernel with one wave per row
//   (205 against 235 us at 8 x 2048 x 1536, 3.5 against 6.9 ms at
//   4 x 65536 x 2048, 370 against 415 us at 16 x 2048 x 1536).
constexpr int64_t kTparMaxRows = 1023;
constexpr int64_t kTparMinLen = 128;
constexpr int64_t kWaveMinLen = 256;
constexpr int64_t kSeqMinRows = 32768;

// Scan kernel shape: G states per thread, NG state groups per channel
// (G * NG >= dstate).  Up to 8 states one group shape covers them; for 9..16
// the choice trades per-thread work against the number of waves: a wave is
// 16 channels x 4 groups (64 lanes), so b * dim * NG / 64 waves share the 1024
// SIMDs.  SSM66_SCAN_KERNEL = "lds1", "lds2" or "lds4" forces G for 9..16
// states (tuning, and tests that cover every instance).
void pick_scan_shape(int64_t batch, int64_t dim, int64_t dstate, int* G, int* NG) {
  if (dstate <= 4) { *G = 1; *NG = 4; return; }
  if (dstate <= 8) { *G = 2; *NG = 4; return; }
  int g = 0;
  if (const char* e = getenv("SSM66_SCAN_KERNEL"))
    if (e[0] == 'l' && e[1] == 'd' && e[2] == 's') g = atoi(e + 3);
  if (g != 1 && g != 2 && g != 4) {
    const int64_t waves4 = batch * dim * 4 / 64;  // waves with G = 4
    g = waves4 >= 2048 ? 4 : (waves4 >= 512 ? 2 : 1);
  }
  *G = g;
  *NG = 16 / g;
}

// Which scan kernel runs (see the crossovers above).  SSM66_SCAN_KERNEL =
// "tpar" forces the time-parallel kernel with four waves per row, "wave" the
// one with one wave per row, "lds*" the sequential one.
enum class ScanKernel { kSequential, kTpar, kWave };

ScanKernel pick_scan_kernel(int64_t batch, int64_t dim, int64_t L, int64_t dstate) {
  // the time-parallel kernels address a 256-token chunk with 32-bit offsets
  if (1024 * dim >= 0xffffffffLL || dstate > 16) return ScanKernel::kSequential;
  if (const char* e = getenv("SSM66_SCAN_KERNEL")) {
    if (e[0] == 't') return ScanKernel::kTpar;
    if (e[0] == 'w') return ScanKernel::kWave;
    if (e[0] == 'l') return ScanKernel::kSequential;
  }
  const int64_t rows = batch * dim;
  if (rows <= kTparMaxRows) return L >= kTparMinLen ? ScanKernel::kTpar : ScanKernel::kSequential;
  if (L < kWaveMinLen || rows >= kSeqMinRows) return ScanKernel::kSequential;
  return ScanKernel::kWave;
}

}  // namespace

extern "C" {

int ssm_abi_version(void) { return SSM_ABI_VERSION; }

const char* ssm_status_string(int status) {
  switch (status) {
    case SSM_OK: return "ok";
    case SSM_ERR_NULL: return "a required pointer is NULL";
    case SSM_ERR_SHAPE: return "invalid shape (negative size, dstate outside [1,16], or overflow)";
    case SSM_ERR_DTYPE: return "unknown io dtype";
    case SSM_ERR_FLAG: return "invalid softplus flag or dt_mode";
    case SSM_ERR_ALIGN: return "pointer not aligned to its element size";
    case SSM_ERR_UNSUPPORTED: return "size not supported by the kernels";
    case SSM_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

static int scan_fwd_impl(const void* u, const void* delta, const float* A, const void* B,
                    const void* C, const float* D, const void* z, const float* delta_bias,
                    int softplus, int dt_mode, const float* h0, const int32_t* seq_lens,
                    const uint8_t* reset, void* y, float* last_state, float* ckpt, int64_t batch,
                    int64_t seqlen, int64_t dim, int64_t dstate, int io_dtype, void* stream) {
  int st = check_common(batch, seqlen, dim, dstate, io_dtype, softplus, dt_mode);
  if (st != SSM_OK) return st;
  const bool has_tokens = batch > 0 && seqlen > 0 && dim > 0;
  const bool has_rows = batch > 0 && dim > 0;
  if (!has_rows) return SSM_OK;
  if (!A) return SSM_ERR_NULL;
  if (has_tokens && (!u || !delta || !B || !C || !y)) return SSM_ERR_NULL;
  if (ckpt && !aligned(ckpt, 4)) return SSM_ERR_ALIGN;
  const size_t es = io_dtype == SSM_BF16 ? 2 : 4;
  const void* io_ptrs[6] = {u, delta, B, C, z, y};
  for (const void* q : io_ptrs)
    if (q && !aligned(q, es)) return SSM_ERR_ALIGN;
  const void* f32_ptrs[6] = {A, D, delta_bias, last_state, h0, seq_lens};
  for (const void* q : f32_ptrs)
    if (q && !aligned(q, 4)) return SSM_ERR_ALIGN;
  // grid size, and 32-bit lane offsets within a chunk (16 groups x dim)
  if (batch * ((dim + 15) / 16) > 0x7fffffff || 16 * dim > 0x7fffffff) return SSM_ERR_UNSUPPORTED;

  ssm66::ScanParams p;
  p.u = u; p.delta = delta; p.A = A; p.B = B; p.C = C; p.D = D; p.z = z;
  p.delta_bias = delta_bias; p.h0 = h0; p.seq_lens = seq_lens; p.reset = reset;
  p.y = y; p.last_state = last_state; p.ckpt = has_tokens ? ckpt : nullptr;
  p.batch = batch; p.L = seqlen; p.dim = dim; p.N = dstate; p.softplus = softplus;
  hipError_t e;
  const ScanKernel kern =
      has_tokens ? pick_scan_kernel(batch, dim, seqlen, dstate) : ScanKernel::kSequential;
  if (kern == ScanKernel::kTpar) {
    e = ssm66::launch_scan_tpar(p, io_dtype, dt_mode == SSM_DT_ZOH, z != nullptr,
                                (hipStream_t)stream);
  } else if (kern == ScanKernel::kWave) {
    e = ssm66::launch_scan_wave(p, io_dtype, dt_mode == SSM_DT_ZOH, z != nullptr,
                                (hipStream_t)stream);
  } else {
    int G, NG;
    pick_scan_shape(batch, dim, dstate, &G, &NG);
    e = ssm66::launch_scan_fwd(p, io_dtype, G, NG, dt_mode == SSM_DT_ZOH, z != nullptr,
                               (hipStream_t)stream);
  }
  return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

int ssm_scan_fwd_ex(const void* u, const void* delta, const float* A, const void* B,
                    const void* C, const float* D, const void* z, const float* delta_bias,
                    int softplus, int dt_mode, const float* h0, const int32_t* seq_lens,
                    const uint8_t* reset, void* y, float* last_state, int64_t batch,
                    int64_t seqlen, int64_t dim, int64_t dstate, int io_dtype, void* stream) {
  return scan_fwd_impl(u, delta, A, B, C, D, z, delta_bias, softplus, dt_mode, h0, seq_lens, reset,
                       y, last_state, nullptr, batch, seqlen, dim, dstate, io_dtype, stream);
}

const char* ssm_scan_kernel_name(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate) {
  if (check_common(batch, seqlen, dim, dstate, SSM_F32, 0, SSM_DT_ZOH) != SSM_OK) return "invalid shape";
  if (batch == 0 || seqlen == 0 || dim == 0) return "none (no tokens)";
  switch (pick_scan_kernel(batch, dim, seqlen, dstate)) {
    case ScanKernel::kTpar: return "scan_tpar_kernel (time-parallel, four waves per row)";
    case ScanKernel::kWave: return "scan_wave_kernel (time-parallel, one wave per row)";
    default: break;
  }
  int G, NG;
  pick_scan_shape(batch, dim, dstate, &G, &NG);
  if (G == 4) return "scan_fwd_kernel (sequential, 4 states per lane)";
  if (G == 2) return "scan_fwd_kernel (sequential, 2 states per lane)";
  return "scan_fwd_kernel (sequential, 1 state per lane)";
}

size_t ssm_scan_ckpt_size(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate) {
  if (check_common(batch, seqlen, dim, dstate, SSM_F32, 0, SSM_DT_ZOH) != SSM_OK) return 0;
  return ssm66::scan_bwd_ckpt_bytes(batch, seqlen, dim, dstate);
}

int ssm_scan_fwd_ckpt(const void* u, const void* delta, const float* A, const void* B,
                      const void* C, const float* D, const void* z, const float* delta_bias,
                      int softplus, int dt_mode, const float* h0, void* y, float* last_state,
                      float* ckpt, int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                      int io_dtype, void* stream) {
  if (seqlen > 0 && batch > 0 && dim > 0 && !ckpt) return SSM_ERR_NULL;
  return scan_fwd_impl(u, delta, A, B, C, D, z, delta_bias, softplus, dt_mode, h0, nullptr,
                       nullptr, y, last_state, ckpt, batch, seqlen, dim, dstate, io_dtype, stream);
}

int ssm_scan_fwd(const void* u, const void* delta, const float* A, const void* B, const void* C,
                 const float* D, const void* z, const float* delta_bias, int softplus,
                 int dt_mode, void* y, float* last_state, int64_t batch, int64_t seqlen,
                 int64_t dim, int64_t dstate, int io_dtype, void* stream) {
  return ssm_scan_fwd_ex(u, delta, A, B, C, D, z, delta_bias, softplus, dt_mode, nullptr, nullptr,
                         nullptr, y, last_state, batch, seqlen, dim, dstate, io_dtype, stream);
}

int ssm_step(float* state, const void* u, const void* delta, const float* A, const void* B,
             const void* C, const float* D, const void* z, const float* delta_bias, int softplus,
             int dt_mode, void* y, int64_t batch, int64_t dim, int64_t dstate, int io_dtype,
             void* stream) {
  int st = check_common(batch, 1, dim, dstate, io_dtype, softplus, dt_mode);
  if (st != SSM_OK) return st;
  if (batch == 0 || dim == 0) return SSM_OK;
  if (!state || !u || !delta || !A || !B || !C || !y) return SSM_ERR_NULL;
  const size_t es = io_dtype == SSM_BF16 ? 2 : 4;
  const void* io_ptrs[6] = {u, delta, B, C, z, y};
  for (const void* q : io_ptrs)
    if (q && !aligned(q, es)) return SSM_ERR_ALIGN;
  const void* f32_ptrs[4] = {state, A, D, delta_bias};
  for (const void* q : f32_ptrs)
    if (q && !aligned(q, 4)) return SSM_ERR_ALIGN;
  int64_t threads;
  if (!mul3(batch, dim, 4, &threads) || (threads + 255) / 256 > 0x7fffffff)
    return SSM_ERR_UNSUPPORTED;

  ssm66::StepParams p;
  p.state = state; p.u = u; p.delta = delta; p.A = A; p.B = B; p.C = C; p.D = D; p.z = z;
  p.delta_bias = delta_bias; p.y = y; p.batch = batch; p.dim = dim; p.N = dstate;
  p.softplus = softplus;
  hipError_t e = ssm66::launch_step(p, io_dtype, dt_mode == SSM_DT_ZOH, z != nullptr,
                                    (hipStream_t)stream);
  return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

size_t ssm_scan_bwd_workspace_size(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate) {
  if (check_common(batch, seqlen, dim, dstate, SSM_F32, 0, SSM_DT_ZOH) != SSM_OK) return 0;
  return ssm66::scan_bwd_workspace_bytes(batch, seqlen, dim, dstate);
}

int ssm_scan_bwd_ex(const void* u, const void* delta, const float* A, const void* B,
                    const void* C, const float* D, const void* z, const float* delta_bias,
                    int softplus, int dt_mode, const float* h0, const void* dy,
                    const float* dlast_state, void* du, void* ddelta, float* dA, void* dB,
                    void* dC, float* dD, void* dz, float* ddelta_bias, float* dh0,
                    const float* ckpt, void* workspace, size_t workspace_bytes, int64_t batch,
                    int64_t seqlen, int64_t dim, int64_t dstate, int io_dtype, void* stream) {
  int st = check_common(batch, seqlen, dim, dstate, io_dtype, softplus, dt_mode);
  if (st != SSM_OK) return st;
  if (batch == 0 || dim == 0) return SSM_OK;
  if (!A || !dA) return SSM_ERR_NULL;
  const bool has_tokens = seqlen > 0;
  if (has_tokens && (!u || !delta || !B || !C || !dy || !du || !ddelta || !dB || !dC))
    return SSM_ERR_NULL;
  if (z && !dz) return SSM_ERR_NULL;  // the gate's gradient is part of the result
  if (!workspace) return SSM_ERR_NULL;
  if (workspace_bytes < ssm66::scan_bwd_workspace_bytes(batch, seqlen, dim, dstate))
    return SSM_ERR_SHAPE;
  const size_t es = io_dtype == SSM_BF16 ? 2 : 4;
  const void* io_ptrs[11] = {u, delta, B, C, z, dy, du, ddelta, dB, dC, dz};
  for (const void* q : io_ptrs)
    if (q && !aligned(q, es)) return SSM_ERR_ALIGN;
  const void* f32_ptrs[11] = {A, D, delta_bias, h0, dlast_state, dA, dD, ddelta_bias, dh0,
                              ckpt, workspace};
  for (const void* q : f32_ptrs)
    if (q && !aligned(q, 4)) return SSM_ERR_ALIGN;
  if (!aligned(workspace, 256)) return SSM_ERR_ALIGN;
  if (batch * ((dim + 15) / 16) > 0x7fffffff) return SSM_ERR_UNSUPPORTED;

  ssm66::ScanBwdParams p;
  p.u = u; p.delta = delta; p.B = B; p.C = C; p.z = z; p.dy = dy;
  p.A = A; p.D = D; p.delta_bias = delta_bias; p.h0 = h0; p.dlast = dlast_state;
  p.du = du; p.ddelta = ddelta; p.dB = dB; p.dC = dC; p.dz = dz;
  p.dA = dA; p.dD = dD; p.ddelta_bias = ddelta_bias; p.dh0 = dh0;
  p.workspace = workspace;
  p.ckpt = ckpt;
  p.batch = batch; p.L = seqlen; p.dim = dim; p.N = dstate; p.softplus = softplus;
  const hipError_t e = ssm66::launch_scan_bwd(p, io_dtype, dt_mode == SSM_DT_ZOH, z != nullptr,
                                              (hipStream_t)stream);
  return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

int ssm_scan_bwd(const void* u, const void* delta, const float* A, const void* B, const void* C,
                 const float* D, const void* z, const float* delta_bias, int softplus,
                 int dt_mode, const float* h0, const void* dy, const float* dlast_state,
                 void* du, void* ddelta, float* dA, void* dB, void* dC, float* dD, void* dz,
                 float* ddelta_bias, float* dh0, void* workspace, size_t workspace_bytes,
                 int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int io_dtype,
                 void* stream) {
  return ssm_scan_bwd_ex(u, delta, A, B, C, D, z, delta_bias, softplus, dt_mode, h0, dy,
                         dlast_state, du, ddelta, dA, dB, dC, dD, dz, ddelta_bias, dh0, nullptr,
                         workspace, workspace_bytes, batch, seqlen, dim, dstate, io_dtype, stream);
}

int ssm_ssd_fwd(const void* x, const float* dt, const float* A, const void* B, const void* C,
                const float* D, const void* z, const float* dt_bias, int softplus, int dt_mode,
                const float* h0, void* y, float* last_state, int64_t batch, int64_t seqlen,
                int64_t nheads, int64_t headdim, int64_t dstate, int io_dtype, void* stream) {
  if (batch < 0 || seqlen < 0 || nheads < 0 || headdim < 1 || dstate < 1) return SSM_ERR_SHAPE;
  if (io_dtype != SSM_F32 && io_dtype != SSM_BF16) return SSM_ERR_DTYPE;
  if (softplus != 0 && softplus != 1) return SSM_ERR_FLAG;
  if (dt_mode != SSM_DT_ZOH && dt_mode != SSM_DT_EULER) return SSM_ERR_FLAG;
  int64_t tmp;
  if (!mul3(batch, seqlen, nheads * headdim, &tmp) || !mul3(batch, seqlen, dstate, &tmp) ||
      !mul3(batch, nheads * headdim, dstate, &tmp))
    return SSM_ERR_SHAPE;
  if (batch == 0 || nheads == 0) return SSM_OK;
  if (!A) return SSM_ERR_NULL;
  if (seqlen > 0 && (!x || !dt || !B || !C || !y)) return SSM_ERR_NULL;
  // the MFMA kernel: bf16 operands, 64 channels per head, 64 or 128 states
  if (io_dtype != SSM_BF16 || headdim != 64 || (dstate != 64 && dstate != 128))
    return SSM_ERR_UNSUPPORTED;
  const void* v16[5] = {x, z, y, B, C};
  for (const void* q : v16)
    if (q && !aligned(q, 16)) return SSM_ERR_ALIGN;
  const void* f32_ptrs[7] = {dt, A, D, dt_bias, h0, last_state, nullptr};
  for (const void* q : f32_ptrs)
    if (q && !aligned(q, 4)) return SSM_ERR_ALIGN;
  if (batch * nheads > 0x7fffffff / 4) return SSM_ERR_UNSUPPORTED;  // 4 blocks per head

  ssm66::SSDParams p;
  p.x = x; p.B = B; p.C = C; p.z = z; p.dt = dt; p.A = A; p.D = D; p.dt_bias = dt_bias;
  p.h0 = h0; p.y = y; p.last_state = last_state;
  p.batch = batch; p.L = seqlen; p.nheads = nheads; p.P = headdim; p.N = dstate;
  p.softplus = softplus;
  const hipError_t e = ssm66::launch_ssd_fwd(p, dt_mode == SSM_DT_ZOH, z != nullptr,
                                             (hipStream_t)stream);
  return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

int ssm_conv1d_fwd(const void* x, const float* weight, const float* bias, int silu,
                   const void* window_in, const int32_t* seq_lens, const uint8_t* reset,
                   void* out, void* window_out, int64_t batch, int64_t seqlen, int64_t dim,
                   int64_t width, int io_dtype, void* stream) {
  if (batch < 0 || seqlen < 0 || dim < 0) return SSM_ERR_SHAPE;
  if (width < 1 || width > 4) return SSM_ERR_SHAPE;
  if (io_dtype != SSM_F32 && io_dtype != SSM_BF16) return SSM_ERR_DTYPE;
  if (silu != 0 && silu != 1) return SSM_ERR_FLAG;
  int64_t tmp;
  if (!mul3(batch, seqlen, dim, &tmp) || !mul3(batch, width, dim, &tmp)) return SSM_ERR_SHAPE;
  if (batch == 0 || dim == 0) return SSM_OK;
  if (!weight) return SSM_ERR_NULL;
  if (seqlen > 0 && (!x || !out)) return SSM_ERR_NULL;
  const size_t es = io_dtype == SSM_BF16 ? 2 : 4;
  const void* io_ptrs[4] = {x, out, window_in, window_out};
  for (const void* q : io_ptrs)
    if (q && !aligned(q, es)) return SSM_ERR_ALIGN;
  const void* f32_ptrs[3] = {weight, bias, seq_lens};
  for (const void* q : f32_ptrs)
    if (q && !aligned(q, 4)) return SSM_ERR_ALIGN;
  // grid: channel vectors in x, 64-token runs in y, batch in z
  if ((seqlen + 63) / 64 > 65535 || batch > 65535 || dim / 64 + 1 > 0x7fffffff)
    return SSM_ERR_UNSUPPORTED;
  bool vec4 = dim % 4 == 0;
  for (const void* q : io_ptrs)
    if (q && !aligned(q, 4 * es)) vec4 = false;

  ssm66::ConvParams p;
  p.x = x; p.w = weight; p.bias = bias; p.state_in = window_in; p.seq_lens = seq_lens;
  p.reset = reset; p.out = out; p.state_out = window_out;
  p.batch = batch; p.L = seqlen; p.dim = dim; p.k = width; p.silu = silu;
  const hipError_t e = ssm66::launch_conv1d(p, io_dtype, vec4, false, (hipStream_t)stream);
  return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

int ssm_conv1d_step(void* window, const void* x, const float* weight, const float* bias,
                    int silu, void* out, int64_t batch, int64_t dim, int64_t width, int io_dtype,
                    void* stream) {
  if (batch < 0 || dim < 0) return SSM_ERR_SHAPE;
  if (width < 1 || width > 4) return SSM_ERR_SHAPE;
  if (io_dtype != SSM_F32 && io_dtype != SSM_BF16) return SSM_ERR_DTYPE;
  if (silu != 0 && silu != 1) return SSM_ERR_FLAG;
  int64_t tmp;
  if (!mul3(batch, width, dim, &tmp)) return SSM_ERR_SHAPE;
  if (batch == 0 || dim == 0) return SSM_OK;
  if (!weight || !x || !out || (width > 1 && !window)) return SSM_ERR_NULL;
  const size_t es = io_dtype == SSM_BF16 ? 2 : 4;
  const void* io_ptrs[3] = {x, out, window};
  for (const void* q : io_ptrs)
    if (q && !aligned(q, es)) return SSM_ERR_ALIGN;
  if (!aligned(weight, 4) || (bias && !aligned(bias, 4))) return SSM_ERR_ALIGN;
  if ((batch * dim + 255) / 256 > 0x7fffffff) return SSM_ERR_UNSUPPORTED;
  bool vec4 = dim % 4 == 0;
  for (const void* q : io_ptrs)
    if (q && !aligned(q, 4 * es)) vec4 = false;

  ssm66::ConvParams p;
  p.x = x; p.w = weight; p.bias = bias; p.state_in = nullptr; p.seq_lens = nullptr;
  p.reset = nullptr; p.out = out; p.state_out = window;
  p.batch = batch; p.L = 1; p.dim = dim; p.k = width; p.silu = silu;
  const hipError_t e = ssm66::launch_conv1d(p, io_dtype, vec4, true, (hipStream_t)stream);
  return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

}  // extern "C"
