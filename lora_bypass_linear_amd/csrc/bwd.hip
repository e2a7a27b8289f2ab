// bwd.hip -- the transposed copies the LoRA-bypass backward contracts over
// tokens with.  dDown = gh_r^T . x_c and dUp = scale * dy_c^T . h_r sum over
// the token index, which is the row index of x, dy, h_r and gh_r; the GEMM
// reads both operands along their rows, so those four (and W for
// dx = dy_c . W_c) are first copied transposed, rounded to the compute dtype,
// with zero padding to 8-element rows.
#include "bwd.h"
#include "lyc_device.h"

namespace lyc {

template <class T>
__device__ __forceinline__ float widen_t(T v, int dt) {
    if constexpr (sizeof(T) == 4) return __builtin_bit_cast(float, v);
    else return dt == DT_F16 ? f16_to_f32(v) : bf16_to_f32(v);
}

// One 64 x 64 tile per workgroup through LDS: the reads run along source
// rows and the writes along destination rows (64 consecutive elements per
// wave instruction on both sides).
template <class T>
__global__ __launch_bounds__(256) void transpose_kernel(TransposeParams p, int64_t tiles_r) {
    __shared__ float t[64][65];
    const int tid = threadIdx.x, l = tid & 63, g = tid >> 6;
    const int64_t r0 = ((int64_t)blockIdx.x % tiles_r) * 64, c0 = ((int64_t)blockIdx.x / tiles_r) * 64;
    const T* src = (const T*)p.src;
    // loads: 16 rows per thread (g, g+4, ...), column l; clamped, then masked
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int64_t r = r0 + g + 4 * i, c = c0 + l;
        const bool ok = r < p.rows && c < p.cols;
        v[i] = widen_t(src[ok ? r * p.cols + c : 0], p.src_dt);
        v[i] = ok ? v[i] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) t[g + 4 * i][l] = v[i];
    __syncthreads();
    // stores: destination row c0 + g + 4i, column r0 + l
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int64_t c = c0 + g + 4 * i, r = r0 + l;
        if (c >= p.cols_pad || r >= p.rows_pad) continue;
        const float x = t[l][g + 4 * i];
        const int64_t at = c * p.rows_pad + r;
        if (p.c_dt == DT_F32) ((float*)p.dst)[at] = x;
        else ((uint16_t*)p.dst)[at] = p.c_dt == DT_F16 ? f32_to_f16(x) : f32_to_bf16(x);
    }
}

hipError_t launch_transpose(const TransposeParams& p, hipStream_t s) {
    if (p.rows_pad <= 0 || p.cols_pad <= 0) return hipSuccess;
    const int64_t tr = (p.rows_pad + 63) / 64, tc = (p.cols_pad + 63) / 64;
    const dim3 grid((unsigned)(tr * tc));
    if (p.src_dt == DT_F32) hipLaunchKernelGGL(transpose_kernel<uint32_t>, grid, dim3(256), 0, s, p, tr);
    else hipLaunchKernelGGL(transpose_kernel<uint16_t>, grid, dim3(256), 0, s, p, tr);
    return hipGetLastError();
}

}  // namespace lyc
