// kq_calib.hpp -- host-side launcher of the calibration kernels (kq_calib.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kq {

// kind: KQ_CALIB_*; *work receives the launch's work (int8 ops, fp32 flops or
// bytes read)
hipError_t launch_calib(int kind, int param, const void *buf, int64_t bytes, int num_cus,
                        double *work, hipStream_t stream);

}  // namespace kq
