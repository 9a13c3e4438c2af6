// ssm_api.hip -- the C ABI declared in include/ssm66.h.
//
// Argument validation runs before any HIP call, so an invalid call returns its
// status without touching a device and with nothing enqueued.  A valid call
// chooses a kernel instance and enqueues one launch on the caller's stream.
#include <stdint.h>

#include <mutex>
#include <string>

#include "../../include/ssm66.h"
#include "ssm_launch.h"

namespace {

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// a * b * c for non-negative a, b, c without int64 overflow; false on
// overflow (each partial product fits in 128 bits)
bool mul3(int64_t a, int64_t b, int64_t c, int64_t* out) {
  const __int128 ab = (__int128)a * b;
  if (ab > INT64_MAX) return false;
  const __int128 r = ab * c;
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

// Kernel choice, from sweeps on MI355X (bf16, N 16, ZOH, gate; kernel times):
// - fewer than 1024 (batch x channel) rows and at least 128 tokens: the
//   time-parallel kernel with four waves per row (88 against 153 us for one
//   wave per row at 1 x 8192 x 256; slower from 1024 rows: 52 against 39 us
//   at 1 x 2048 x 1024);
// - 12288 rows or more (three waves per SIMD with four rows per wave) and at
//   least 128 tokens: the time-parallel kernel with 16 lanes per row, eight
//   tokens per lane with bf16 io and no lengths or document starts, four
//   otherwise (with four: 161 against 167 us for one wave per row at
//   8 x 2048 x 1536; 391 against 448, and 425 for the sequential kernel, at
//   8 x 2048 x 4096; 760 against 821 for the sequential kernel at
//   16 x 2048 x 4096; 17 against 22 us for the sequential kernel at
//   8 x 128 x 1536, even at 8 x 64 x 1536; with eight: 146.5 and 357 us at
//   8 x 2048 x 1536 and 8 x 2048 x 4096);
// - from 8192 rows when the eight-token kernel takes the call (bf16 io, 16
//   states, a width that is a multiple of 16, no lengths or document starts)
//   and at least 128 tokens: that kernel (3.01 against 3.32 ms for one wave per
//   row under ZOH, 2.61 against 2.96 ms under Euler, at 4 x 65536 x 2048);
// - between 1024 and 12288 rows and at least 256 tokens: the time-parallel
//   kernel with one wave per row (146 against 160 us for 16 lanes per row at
//   2 x 2048 x 5120; 3.5 against 6.9 ms for the sequential kernel at
//   4 x 65536 x 2048);
// - shorter sequences: the sequential kernel (19 against 30 us for one wave
//   per row at 8 x 64 x 1536).
constexpr int64_t kTparMaxRows = 1023;
constexpr int64_t kTparMinLen = 128;
constexpr int64_t kWaveMinLen = 256;
constexpr int64_t kWave4MinRows = 12288;
constexpr int64_t kWave8MinRows = 8192;
constexpr int64_t kWave4MinLen = 128;

// Scan kernel shape: G states per thread, NG state groups per channel
// (G * NG >= dstate).  Up to 8 states one group shape covers them; for 9..16
// the choice trades per-thread work against the number of waves: a wave is
// 16 channels x 4 groups (64 lanes), so b * dim * NG / 64 waves share the 1024
// SIMDs.  forced_g (1, 2 or 4; 0 = choose) fixes G for 9..16 states.
void pick_scan_shape(int64_t batch, int64_t dim, int64_t dstate, int forced_g, int* G, int* NG) {
  if (dstate <= 4) { *G = 1; *NG = 4; return; }
  if (dstate <= 8) { *G = 2; *NG = 4; return; }
  int g = forced_g;
  if (g != 1 && g != 2 && g != 4) {
    const int64_t waves4 = batch * dim * 4 / 64;  // waves with G = 4
    g = waves4 >= 2048 ? 4 : (waves4 >= 512 ? 2 : 1);
  }
  *G = g;
  *NG = 16 / g;
}

// Which scan kernel runs (see the crossovers above).
enum class ScanKernel { kSequential, kTpar, kWave, kWave4 };

// the time-parallel kernels address a 256-token chunk of up to 4-byte
// elements with 32-bit offsets: 1024 dim < 2^32 - 1
bool tpar_fits(int64_t dim) { return dim < ((int64_t)1 << 22); }

// eight: the call is one the eight-token kernel takes (bf16 io, 16 states, a
// width that is a multiple of 16, no lengths or document starts).
ScanKernel pick_scan_kernel(int64_t batch, int64_t dim, int64_t L, int64_t dstate, bool eight) {
  if (!tpar_fits(dim) || dstate > 16) return ScanKernel::kSequential;
  const int64_t rows = batch * dim;
  if (rows <= kTparMaxRows) return L >= kTparMinLen ? ScanKernel::kTpar : ScanKernel::kSequential;
  if (rows >= (eight ? kWave8MinRows : kWave4MinRows))
    return L >= kWave4MinLen ? ScanKernel::kWave4 : ScanKernel::kSequential;
  return L >= kWaveMinLen ? ScanKernel::kWave : ScanKernel::kSequential;
}

// Grid of the chosen kernel within the launch limit (one block per 16
// channels for the sequential kernel and for 16 lanes per row, per 8 for one
// wave per row, per row for four waves per row).
bool grid_fits(ScanKernel k, int64_t batch, int64_t dim) {
  const int64_t per = k == ScanKernel::kWave ? 8 : (k == ScanKernel::kTpar ? 1 : 16);
  const __int128 blocks = (__int128)batch * ((dim + per - 1) / per);
  return blocks <= 0x7fffffff;
}

// The backward pass's workspace for callers that cannot allocate
// (ssm_scan_bwd_noalloc): a fixed array in device memory, one copy per GPU the
// library runs on, held until the process ends.  Host code never passes the
// array's name to a kernel (on the host it only stands for the symbol): each
// device's address comes from hipGetSymbolAddress, once, with that device
// current, and is kept here.
constexpr size_t kScratchBytes = (size_t)SSM_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // per device; set once under g_scratch_mu

// The current device's address of `scratch`: SSM_OK, or SSM_ERR_HIP if the
// runtime cannot name the device or the symbol, SSM_ERR_UNSUPPORTED for a
// device index past the table.
int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SSM_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return SSM_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return SSM_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return SSM_OK;
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

// kernel: SSM_SCAN_KERNEL_AUTO, or one of the forced choices of
// ssm_scan_fwd_kernel (validated by the caller).
static int scan_fwd_impl(int kernel, const void* u, const void* delta, const float* A,
                         const void* B, const void* C, const float* D, const void* z,
                         const float* delta_bias, int softplus, int dt_mode, const float* h0,
                         const int32_t* seq_lens, const uint8_t* reset, void* y,
                         float* last_state, float* ckpt, int64_t batch, int64_t seqlen,
                         int64_t dim, int64_t dstate, int io_dtype, void* stream) {
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
  // the sequential kernel's 32-bit lane offsets within a chunk (16 groups x dim)
  if (dim > 0x7fffffff / 16) return SSM_ERR_UNSUPPORTED;

  ScanKernel kern = ScanKernel::kSequential;
  int forced_g = 0;
  if (!has_tokens) {
    kern = ScanKernel::kSequential;  // writes the initial state only
  } else if (kernel == SSM_SCAN_KERNEL_AUTO) {
    const bool eight = io_dtype == SSM_BF16 && dstate == 16 && dim % 16 == 0 && !seq_lens && !reset;
    kern = pick_scan_kernel(batch, dim, seqlen, dstate, eight);
  } else if (kernel == SSM_SCAN_KERNEL_TPAR || kernel == SSM_SCAN_KERNEL_WAVE ||
             kernel == SSM_SCAN_KERNEL_WAVE4) {
    if (!tpar_fits(dim)) return SSM_ERR_UNSUPPORTED;
    kern = kernel == SSM_SCAN_KERNEL_TPAR ? ScanKernel::kTpar
                                          : (kernel == SSM_SCAN_KERNEL_WAVE ? ScanKernel::kWave : ScanKernel::kWave4);
  } else {
    forced_g = kernel == SSM_SCAN_KERNEL_SEQ1 ? 1 : (kernel == SSM_SCAN_KERNEL_SEQ2 ? 2 : 4);
  }
  if (!grid_fits(kern, batch, dim)) return SSM_ERR_UNSUPPORTED;

  ssm66::ScanParams p;
  p.u = u; p.delta = delta; p.A = A; p.B = B; p.C = C; p.D = D; p.z = z;
  p.delta_bias = delta_bias; p.h0 = h0; p.seq_lens = seq_lens; p.reset = reset;
  p.y = y; p.last_state = last_state; p.ckpt = has_tokens ? ckpt : nullptr;
  p.batch = batch; p.L = seqlen; p.dim = dim; p.N = dstate; p.softplus = softplus;
  hipError_t e;
  if (kern == ScanKernel::kTpar) {
    e = ssm66::launch_scan_tpar(p, io_dtype, dt_mode == SSM_DT_ZOH, z != nullptr,
                                (hipStream_t)stream);
  } else if (kern == ScanKernel::kWave || kern == ScanKernel::kWave4) {
    e = ssm66::launch_scan_wave(p, io_dtype, dt_mode == SSM_DT_ZOH, z != nullptr,
                                kern == ScanKernel::kWave4 ? 4 : 1, (hipStream_t)stream);
  } else {
    int G, NG;
    pick_scan_shape(batch, dim, dstate, forced_g, &G, &NG);
    e = ssm66::launch_scan_fwd(p, io_dtype, G, NG, dt_mode == SSM_DT_ZOH, z != nullptr,
                               (hipStream_t)stream);
  }
  return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

int ssm_scan_fwd_kernel(int kernel, const void* u, const void* delta, const float* A,
                        const void* B, const void* C, const float* D, const void* z,
                        const float* delta_bias, int softplus, int dt_mode, const float* h0,
                        const int32_t* seq_lens, const uint8_t* reset, void* y,
                        float* last_state, float* ckpt, int64_t batch, int64_t seqlen,
                        int64_t dim, int64_t dstate, int io_dtype, void* stream) {
  if (kernel < SSM_SCAN_KERNEL_AUTO || kernel > SSM_SCAN_KERNEL_WAVE4) return SSM_ERR_FLAG;
  return scan_fwd_impl(kernel, u, delta, A, B, C, D, z, delta_bias, softplus, dt_mode, h0,
                       seq_lens, reset, y, last_state, ckpt, batch, seqlen, dim, dstate, io_dtype,
                       stream);
}

int ssm_scan_fwd_ex(const void* u, const void* delta, const float* A, const void* B,
                    const void* C, const float* D, const void* z, const float* delta_bias,
                    int softplus, int dt_mode, const float* h0, const int32_t* seq_lens,
                    const uint8_t* reset, void* y, float* last_state, int64_t batch,
                    int64_t seqlen, int64_t dim, int64_t dstate, int io_dtype, void* stream) {
  return scan_fwd_impl(SSM_SCAN_KERNEL_AUTO, u, delta, A, B, C, D, z, delta_bias, softplus,
                       dt_mode, h0, seq_lens, reset, y, last_state, nullptr, batch, seqlen, dim,
                       dstate, io_dtype, stream);
}

// The name of a kernel choice other than the eight-token split below.
static const char* scan_kernel_label(ScanKernel k, int64_t batch, int64_t dim, int64_t dstate) {
  switch (k) {
    case ScanKernel::kTpar: return "scan_tpar_kernel (time-parallel, four waves per row)";
    case ScanKernel::kWave: return "scan_wave_kernel (time-parallel, one wave per row)";
    case ScanKernel::kWave4:
      return "scan_wave8_kernel / scan_wave_kernel (time-parallel, 16 lanes per row; 8 tokens per lane for bf16 "
             "io without lengths or document starts, else 4)";
    default: break;
  }
  int G, NG;
  pick_scan_shape(batch, dim, dstate, 0, &G, &NG);
  if (G == 4) return "scan_fwd_kernel (sequential, 4 states per lane)";
  if (G == 2) return "scan_fwd_kernel (sequential, 2 states per lane)";
  return "scan_fwd_kernel (sequential, 1 state per lane)";
}

const char* ssm_scan_kernel_name(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate) {
  if (check_common(batch, seqlen, dim, dstate, SSM_F32, 0, SSM_DT_ZOH) != SSM_OK) return "invalid shape";
  if (batch == 0 || seqlen == 0 || dim == 0) return "none (no tokens)";
  const bool eight_ok = dstate == 16 && dim % 16 == 0;
  const ScanKernel k = pick_scan_kernel(batch, dim, seqlen, dstate, false);
  const ScanKernel k8 = pick_scan_kernel(batch, dim, seqlen, dstate, eight_ok);
  if (k8 == k) return scan_kernel_label(k, batch, dim, dstate);
  // rows where the choice depends on the call: the eight-token kernel for the
  // calls it takes, the other choice for the rest (C++ initialises these
  // function-local statics once, thread-safely)
  static const std::string prefix =
      "scan_wave8_kernel (time-parallel, 16 lanes per row, 8 tokens per lane) for bf16 io without lengths or "
      "document starts, else ";
  static const std::string one = prefix + scan_kernel_label(ScanKernel::kWave, 0, 0, 0);
  static const std::string seq1 = prefix + "scan_fwd_kernel (sequential, 1 state per lane)";
  static const std::string seq2 = prefix + "scan_fwd_kernel (sequential, 2 states per lane)";
  static const std::string seq4 = prefix + "scan_fwd_kernel (sequential, 4 states per lane)";
  if (k == ScanKernel::kWave) return one.c_str();
  // otherwise the sequential kernel (the eight-token kernel needs 8192 rows,
  // past the four-waves-per-row range)
  int G, NG;
  pick_scan_shape(batch, dim, dstate, 0, &G, &NG);
  return G == 4 ? seq4.c_str() : (G == 2 ? seq2.c_str() : seq1.c_str());
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
  return scan_fwd_impl(SSM_SCAN_KERNEL_AUTO, u, delta, A, B, C, D, z, delta_bias, softplus,
                       dt_mode, h0, nullptr, nullptr, y, last_state, ckpt, batch, seqlen, dim,
                       dstate, io_dtype, stream);
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

// workspace == NULL with use_scratch: the library's static scratch (checked
// against its size before any HIP call).
static int scan_bwd_impl(const void* u, const void* delta, const float* A, const void* B,
                         const void* C, const float* D, const void* z, const float* delta_bias,
                         int softplus, int dt_mode, const float* h0, const int32_t* seq_lens,
                         const uint8_t* reset, const void* dy,
                         const float* dlast_state, void* du, void* ddelta, float* dA, void* dB,
                         void* dC, float* dD, void* dz, float* ddelta_bias, float* dh0,
                         const float* ckpt, void* workspace, size_t workspace_bytes,
                         bool use_scratch, int64_t batch, int64_t seqlen, int64_t dim,
                         int64_t dstate, int io_dtype, void* stream) {
  int st = check_common(batch, seqlen, dim, dstate, io_dtype, softplus, dt_mode);
  if (st != SSM_OK) return st;
  if (batch == 0 || dim == 0) return SSM_OK;
  if (!A || !dA) return SSM_ERR_NULL;
  const bool has_tokens = seqlen > 0;
  if (has_tokens && (!u || !delta || !B || !C || !dy || !du || !ddelta || !dB || !dC))
    return SSM_ERR_NULL;
  if (z && !dz) return SSM_ERR_NULL;  // the gate's gradient is part of the result
  const size_t need = ssm66::scan_bwd_workspace_bytes(batch, seqlen, dim, dstate);
  if (use_scratch) {
    if (need > kScratchBytes) return SSM_ERR_UNSUPPORTED;
  } else {
    if (!workspace) return SSM_ERR_NULL;
    if (workspace_bytes < need) return SSM_ERR_SHAPE;
  }
  const size_t es = io_dtype == SSM_BF16 ? 2 : 4;
  const void* io_ptrs[11] = {u, delta, B, C, z, dy, du, ddelta, dB, dC, dz};
  for (const void* q : io_ptrs)
    if (q && !aligned(q, es)) return SSM_ERR_ALIGN;
  const void* f32_ptrs[12] = {A, D, delta_bias, h0, dlast_state, dA, dD, ddelta_bias, dh0,
                              ckpt, workspace, seq_lens};
  for (const void* q : f32_ptrs)
    if (q && !aligned(q, 4)) return SSM_ERR_ALIGN;
  if (workspace && !aligned(workspace, 256)) return SSM_ERR_ALIGN;
  if (batch * ((dim + 15) / 16) > 0x7fffffff) return SSM_ERR_UNSUPPORTED;
  if (use_scratch) {  // validation is done: the first HIP call
    st = scratch_address(&workspace);
    if (st != SSM_OK) return st;
  }

  ssm66::ScanBwdParams p;
  p.u = u; p.delta = delta; p.B = B; p.C = C; p.z = z; p.dy = dy;
  p.A = A; p.D = D; p.delta_bias = delta_bias; p.h0 = h0; p.dlast = dlast_state;
  p.seq_lens = seq_lens; p.reset = reset;
  p.du = du; p.ddelta = ddelta; p.dB = dB; p.dC = dC; p.dz = dz;
  p.dA = dA; p.dD = dD; p.ddelta_bias = ddelta_bias; p.dh0 = dh0;
  p.workspace = workspace;
  p.ckpt = ckpt;
  p.batch = batch; p.L = seqlen; p.dim = dim; p.N = dstate; p.softplus = softplus;
  const hipError_t e = ssm66::launch_scan_bwd(p, io_dtype, dt_mode == SSM_DT_ZOH, z != nullptr,
                                              (hipStream_t)stream);
  return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

int ssm_scan_bwd_ex(const void* u, const void* delta, const float* A, const void* B,
                    const void* C, const float* D, const void* z, const float* delta_bias,
                    int softplus, int dt_mode, const float* h0, const int32_t* seq_lens,
                    const uint8_t* reset, const void* dy, const float* dlast_state, void* du,
                    void* ddelta, float* dA, void* dB, void* dC, float* dD, void* dz,
                    float* ddelta_bias, float* dh0, const float* ckpt, void* workspace,
                    size_t workspace_bytes, int64_t batch, int64_t seqlen, int64_t dim,
                    int64_t dstate, int io_dtype, void* stream) {
  return scan_bwd_impl(u, delta, A, B, C, D, z, delta_bias, softplus, dt_mode, h0, seq_lens,
                       reset, dy,
                       dlast_state, du, ddelta, dA, dB, dC, dD, dz, ddelta_bias, dh0, ckpt,
                       workspace, workspace_bytes, false, batch, seqlen, dim, dstate, io_dtype,
                       stream);
}

int ssm_scan_bwd_noalloc(const void* u, const void* delta, const float* A, const void* B,
                         const void* C, const float* D, const void* z, const float* delta_bias,
                         int softplus, int dt_mode, const float* h0, const int32_t* seq_lens,
                         const uint8_t* reset, const void* dy, const float* dlast_state,
                         void* du, void* ddelta, float* dA, void* dB, void* dC, float* dD,
                         void* dz, float* ddelta_bias, float* dh0, const float* ckpt,
                         int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                         int io_dtype, void* stream) {
  return scan_bwd_impl(u, delta, A, B, C, D, z, delta_bias, softplus, dt_mode, h0, seq_lens,
                       reset, dy,
                       dlast_state, du, ddelta, dA, dB, dC, dD, dz, ddelta_bias, dh0, ckpt,
                       nullptr, 0, true, batch, seqlen, dim, dstate, io_dtype, stream);
}

int ssm_scan_bwd(const void* u, const void* delta, const float* A, const void* B, const void* C,
                 const float* D, const void* z, const float* delta_bias, int softplus,
                 int dt_mode, const float* h0, const void* dy, const float* dlast_state,
                 void* du, void* ddelta, float* dA, void* dB, void* dC, float* dD, void* dz,
                 float* ddelta_bias, float* dh0, void* workspace, size_t workspace_bytes,
                 int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int io_dtype,
                 void* stream) {
  return ssm_scan_bwd_ex(u, delta, A, B, C, D, z, delta_bias, softplus, dt_mode, h0, nullptr,
                         nullptr, dy,
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
  int64_t dim, tmp;
  if (!mul3(nheads, headdim, 1, &dim) || !mul3(batch, seqlen, dim, &tmp) ||
      !mul3(batch, seqlen, dstate, &tmp) || !mul3(batch, dim, dstate, &tmp))
    return SSM_ERR_SHAPE;
  if (batch == 0 || nheads == 0) return SSM_OK;
  if (!A) return SSM_ERR_NULL;
  if (seqlen > 0 && (!x || !dt || !B || !C || !y)) return SSM_ERR_NULL;
  // the MFMA kernel: bf16 operands, a multiple of 16 channels per head, 64 or
  // 128 states
  if (io_dtype != SSM_BF16 || headdim % 16 != 0 || (dstate != 64 && dstate != 128))
    return SSM_ERR_UNSUPPORTED;
  const void* v16[5] = {x, z, y, B, C};
  for (const void* q : v16)
    if (q && !aligned(q, 16)) return SSM_ERR_ALIGN;
  const void* f32_ptrs[7] = {dt, A, D, dt_bias, h0, last_state, nullptr};
  for (const void* q : f32_ptrs)
    if (q && !aligned(q, 4)) return SSM_ERR_ALIGN;
  if (batch * nheads > 0x7fffffff / (headdim / 16)) return SSM_ERR_UNSUPPORTED;  // P / 16 blocks per head
  if (dim > ((int64_t)1 << 23)) return SSM_ERR_UNSUPPORTED;  // a chunk's rows addressed in 32 bits

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

static int conv_bwd_shape(int64_t batch, int64_t seqlen, int64_t dim, int64_t width) {
  if (batch < 0 || seqlen < 0 || dim < 0) return SSM_ERR_SHAPE;
  if (width < 1 || width > 4) return SSM_ERR_SHAPE;
  int64_t tmp;
  if (!mul3(batch, seqlen, dim, &tmp) || !mul3(batch, width, dim, &tmp) ||
      !mul3(batch, (seqlen + 127) / 128 + 1, (width + 1) * dim, &tmp))
    return SSM_ERR_SHAPE;
  return SSM_OK;
}

size_t ssm_conv1d_bwd_workspace_size(int64_t batch, int64_t seqlen, int64_t dim, int64_t width) {
  if (conv_bwd_shape(batch, seqlen, dim, width) != SSM_OK) return 0;
  return ssm66::conv1d_bwd_workspace_bytes(batch, seqlen, dim, width);
}

int ssm_conv1d_bwd(const void* x, const float* weight, const float* bias, int silu,
                   const void* window_in, const int32_t* seq_lens, const uint8_t* reset,
                   const void* dout, const void* dwindow_out, void* dx, float* dweight,
                   float* dbias, void* dwindow_in, void* workspace, size_t workspace_bytes,
                   int64_t batch, int64_t seqlen, int64_t dim, int64_t width, int io_dtype,
                   void* stream) {
  int st = conv_bwd_shape(batch, seqlen, dim, width);
  if (st != SSM_OK) return st;
  if (io_dtype != SSM_F32 && io_dtype != SSM_BF16) return SSM_ERR_DTYPE;
  if (silu != 0 && silu != 1) return SSM_ERR_FLAG;
  if (dim == 0) return SSM_OK;
  if (!weight || !dweight) return SSM_ERR_NULL;
  if (seqlen > 0 && (!x || !dout || !dx)) return SSM_ERR_NULL;
  if (width > 1 && window_in && dwindow_in == window_in) return SSM_ERR_FLAG;  // no in-place
  const size_t need = ssm66::conv1d_bwd_workspace_bytes(batch, seqlen, dim, width);
  if (!workspace) return SSM_ERR_NULL;
  if (workspace_bytes < need) return SSM_ERR_SHAPE;
  const size_t es = io_dtype == SSM_BF16 ? 2 : 4;
  const void* io_ptrs[6] = {x, dout, dx, window_in, dwindow_out, dwindow_in};
  for (const void* q : io_ptrs)
    if (q && !aligned(q, es)) return SSM_ERR_ALIGN;
  const void* f32_ptrs[5] = {weight, bias, seq_lens, dweight, dbias};
  for (const void* q : f32_ptrs)
    if (q && !aligned(q, 4)) return SSM_ERR_ALIGN;
  if (!aligned(workspace, 16)) return SSM_ERR_ALIGN;
  // grid: 64 channel vectors in x, 128-token spans in y, batch in z; one
  // sequence's bytes within 32-bit buffer offsets
  if ((seqlen + 127) / 128 > 65535 || batch > 65535 || dim / 64 + 1 > 0x7fffffff)
    return SSM_ERR_UNSUPPORTED;
  if (seqlen * dim > (int64_t)0x7fffffff / (int64_t)es) return SSM_ERR_UNSUPPORTED;
  bool vec4 = dim % 4 == 0;
  for (const void* q : io_ptrs)
    if (q && !aligned(q, 4 * es)) vec4 = false;

  ssm66::ConvBwdParams p;
  p.x = x; p.w = weight; p.bias = bias; p.state_in = window_in; p.seq_lens = seq_lens;
  p.reset = reset; p.dout = dout; p.dstate_out = dwindow_out; p.dx = dx; p.dw = dweight;
  p.dbias = dbias; p.dstate_in = dwindow_in; p.workspace = workspace;
  p.batch = batch; p.L = seqlen; p.dim = dim; p.k = width; p.silu = silu;
  const hipError_t e = ssm66::launch_conv1d_bwd(p, io_dtype, vec4, (hipStream_t)stream);
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
  if (batch * dim > (int64_t)0x7fffffff * 256) return SSM_ERR_UNSUPPORTED;
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

int ssm_alu_probe(int op, float* sink, int64_t blocks, int64_t iters, void* stream) {
  if (op != SSM_PROBE_FMA && op != SSM_PROBE_EXP && op != SSM_PROBE_MIX) return SSM_ERR_FLAG;
  if (blocks < 1 || blocks > 0x7fffffff || iters < 0 || iters > 0x7fffffff) return SSM_ERR_SHAPE;
  if (!sink) return SSM_ERR_NULL;
  if (!aligned(sink, 4)) return SSM_ERR_ALIGN;
  const hipError_t e = ssm66::launch_alu_probe(op, sink, blocks, (int)iters, (hipStream_t)stream);
  return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

}  // extern "C"
