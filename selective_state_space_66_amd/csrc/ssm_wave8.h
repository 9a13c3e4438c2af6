// ssm_wave8.h -- the time-parallel scan with eight tokens per lane
// (scan_wave8.hip): the case it takes, and its launch.
#pragma once

#include <hip/hip_runtime.h>

#include "ssm_launch.h"

namespace ssm66 {

// bf16 io (io_dtype 1), N = 16, no lengths or document starts, dim a
// multiple of 16, the row tensors, B, C and the checkpoints (if any) 16-byte
// aligned, and a grid and chunk offsets within 32 bits
bool scan_wave8_fits(const ScanParams& p, int io_dtype);

// the scan of p (which scan_wave8_fits accepts) on stream
hipError_t launch_scan_wave8(const ScanParams& p, bool zoh, bool gate, hipStream_t stream);

}  // namespace ssm66
