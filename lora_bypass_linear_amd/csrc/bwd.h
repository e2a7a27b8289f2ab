// bwd.h -- host-side launchers of the kernels only the backward uses
// (internal to the library; the public surface is include/lyc.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lyc {

// dst[c][r] = round_c(src[r][c]) for r < rows, c < cols; dst is
// [cols_pad][rows_pad] in the compute dtype, zero outside the source.
struct TransposeParams {
    const void* src;
    int src_dt;
    int64_t rows, cols;          // src [rows][cols], row-major, contiguous
    void* dst;
    int c_dt;
    int64_t rows_pad, cols_pad;  // dst [cols_pad][rows_pad]; rows_pad >= rows, cols_pad >= cols
};
hipError_t launch_transpose(const TransposeParams& p, hipStream_t s);

}  // namespace lyc
