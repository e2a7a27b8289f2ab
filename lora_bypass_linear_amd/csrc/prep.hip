// prep.hip -- operand preparation for the LoRA bypass and the fp32-operand
// casts (master-weight pattern: fp32 storage, 16-bit compute).
//
// Matmul operands enter the contraction in the compute dtype, rounded to
// nearest even from their stored value (LyCORIS "Precision" page, "Dtype
// policy": compute is what the matmul operands are in).  The low-rank factors
// are small (rank x K and N x rank), so they are rewritten once per call into
// compute-dtype copies padded to a rank multiple of 32; the row norms of
// down_c feed the h guard.
#include "kernels.h"
#include "lyc_device.h"

namespace lyc {

__device__ __forceinline__ void store_c(void* dst, int64_t i, float v, int c_dt, double* as_f64) {
    if (c_dt == DT_F32) {
        ((float*)dst)[i] = v;
        *as_f64 = (double)v;
    } else if (c_dt == DT_F16) {
        const uint16_t b = f32_to_f16(v);
        ((uint16_t*)dst)[i] = b;
        *as_f64 = (double)f16_to_f32(b);
    } else {
        const uint16_t b = f32_to_bf16(v);
        ((uint16_t*)dst)[i] = b;
        *as_f64 = (double)bf16_to_f32(b);
    }
}

// blocks [0, r_pad): one row of down each (+ its norm); the rest: up, grid-stride
__global__ __launch_bounds__(256) void prep_kernel(PrepParams p) {
    __shared__ double red[256];
    const int b = blockIdx.x, tid = threadIdx.x;
    if (b == 0 && tid == 0) *p.flagged = 0u;
    if (b < p.r_pad) {
        const int j = b;
        double ss = 0.0;
        for (int64_t k = tid; k < p.K; k += 256) {
            const float v = j < p.rank ? load_as_f32(p.down, p.down_dt, (int64_t)j * p.K + k) : 0.f;
            double c;
            store_c(p.dc, (int64_t)j * p.K + k, v, p.c_dt, &c);
            ss = __builtin_fma(c, c, ss);
        }
        red[tid] = ss;
        __syncthreads();
        for (int o = 128; o > 0; o >>= 1) {
            if (tid < o) red[tid] += red[tid + o];
            __syncthreads();
        }
        if (tid == 0) p.dnorm[j] = __builtin_sqrt(red[0]);
    } else {
        const int64_t total = p.N * (int64_t)p.r_pad;
        const int64_t stride = (int64_t)(gridDim.x - p.r_pad) * 256;
        for (int64_t i = (int64_t)(b - p.r_pad) * 256 + tid; i < total; i += stride) {
            const int64_t n = i / p.r_pad;
            const int j = (int)(i - n * p.r_pad);
            const float v = j < p.rank ? load_as_f32(p.up, p.up_dt, n * p.rank + j) : 0.f;
            double c;
            store_c(p.uc, i, v, p.c_dt, &c);
        }
    }
}

hipError_t launch_prep(const PrepParams& p, hipStream_t s) {
    const int64_t total = p.N * (int64_t)p.r_pad;
    int64_t up_blocks = (total + 255) / 256;
    if (up_blocks > 2048) up_blocks = 2048;
    if (up_blocks < 1) up_blocks = 1;
    hipLaunchKernelGGL(prep_kernel, dim3((unsigned)(p.r_pad + up_blocks)), dim3(256), 0, s, p);
    return hipGetLastError();
}

// fp32 -> 16-bit compute copy (x or W stored in fp32 under a 16-bit policy)
__global__ __launch_bounds__(256) void cast_kernel(const float* __restrict__ src, uint16_t* __restrict__ dst,
                                                   int64_t n, int c_dt) {
    const int64_t n4 = n / 4;
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) {
        const f32x4 v = ((const f32x4*)src)[i];
        uint16_t o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = c_dt == DT_F16 ? f32_to_f16(v[e]) : f32_to_bf16(v[e]);
        ((i32x2*)dst)[i] = i32x2{(int)(o[0] | ((uint32_t)o[1] << 16)), (int)(o[2] | ((uint32_t)o[3] << 16))};
    }
    for (int64_t i = n4 * 4 + (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride)
        dst[i] = c_dt == DT_F16 ? f32_to_f16(src[i]) : f32_to_bf16(src[i]);
}

hipError_t launch_cast(const float* src, void* dst, int64_t n, int c_dt, hipStream_t s) {
    int64_t blocks = (n / 4 + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(cast_kernel, dim3((unsigned)blocks), dim3(256), 0, s, src, (uint16_t*)dst, n, c_dt);
    return hipGetLastError();
}

}  // namespace lyc
