// mfma_probe.hip -- TEST INFRASTRUCTURE.  One MFMA step per wave on given
// operands, so the tests can check, against exact host arithmetic, the lane
// layouts the kernels assume and the rounding error of one step (which sizes
// the h guard).  Every index stays inside the trial's own 16x32 / 32x16 / 16x16
// blocks; the grid has exactly one wave per trial.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

// a: [T][16][32] (row i, k), bt: [T][16][32] (column j, k), c/d: [T][16][16] (i, j)
__global__ __launch_bounds__(64) void probe16(int dt, const uint16_t* a, const uint16_t* bt, const float* c,
                                              float* d, int T) {
    const int t = blockIdx.x, l = threadIdx.x;
    if (t >= T) return;
    const i32x4 av = *(const i32x4*)(a + (size_t)t * 512 + (l & 15) * 32 + 8 * (l >> 4));
    const i32x4 bv = *(const i32x4*)(bt + (size_t)t * 512 + (l & 15) * 32 + 8 * (l >> 4));
    f32x4 acc;
    for (int e = 0; e < 4; ++e) acc[e] = c[(size_t)t * 256 + (4 * (l >> 4) + e) * 16 + (l & 15)];
    if (dt == 1)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, av), __builtin_bit_cast(f16x8, bv), acc, 0, 0, 0);
    else
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, bv), acc, 0, 0, 0);
    for (int e = 0; e < 4; ++e) d[(size_t)t * 256 + (4 * (l >> 4) + e) * 16 + (l & 15)] = acc[e];
}

// fp32: a, bt [T][16][16] (row/column, k); one 16-byte fragment of 4 k values
// per lane (lane group g holds k = 4g .. 4g+3), consumed by four chained
// v_mfma_f32_16x16x4_f32, element e in the e-th instruction.
__global__ __launch_bounds__(64) void probe32(const float* a, const float* bt, const float* c, float* d, int T) {
    const int t = blockIdx.x, l = threadIdx.x;
    if (t >= T) return;
    const f32x4 av = *(const f32x4*)(a + (size_t)t * 256 + (l & 15) * 16 + 4 * (l >> 4));
    const f32x4 bv = *(const f32x4*)(bt + (size_t)t * 256 + (l & 15) * 16 + 4 * (l >> 4));
    f32x4 acc;
    for (int e = 0; e < 4; ++e) acc[e] = c[(size_t)t * 256 + (4 * (l >> 4) + e) * 16 + (l & 15)];
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av.x, bv.x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av.y, bv.y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av.z, bv.z, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av.w, bv.w, acc, 0, 0, 0);
    for (int e = 0; e < 4; ++e) d[(size_t)t * 256 + (4 * (l >> 4) + e) * 16 + (l & 15)] = acc[e];
}

extern "C" int probe_mfma32(const void* a, const void* bt, const void* c, void* d, int T, void* stream) {
    if (T <= 0) return 1;
    hipLaunchKernelGGL(probe32, dim3(T), dim3(64), 0, (hipStream_t)stream, (const float*)a, (const float*)bt,
                       (const float*)c, (float*)d, T);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

extern "C" int probe_mfma16(int dt, const void* a, const void* bt, const void* c, void* d, int T, void* stream) {
    if (T <= 0 || (dt != 1 && dt != 2)) return 1;
    hipLaunchKernelGGL(probe16, dim3(T), dim3(64), 0, (hipStream_t)stream, dt, (const uint16_t*)a,
                       (const uint16_t*)bt, (const float*)c, (float*)d, T);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}
