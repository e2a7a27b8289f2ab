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

// floor(log2 v) of a positive finite fp32 value (subnormals included)
__device__ __forceinline__ int floor_log2(float v) {
    const uint32_t u = __builtin_bit_cast(uint32_t, v);
    const int E = (int)(u >> 23);
    return E > 0 ? E - 127 : (31 - __builtin_clz(u)) - 149;
}

__device__ __forceinline__ void store16(void* dst, int64_t i, float v, int c_dt) {
    ((uint16_t*)dst)[i] = c_dt == DT_F16 ? f32_to_f16(v) : f32_to_bf16(v);
}

// One row of a [rows, K] operand per workgroup of 256 threads; thread t takes
// the 8 consecutive elements k0 + 8t .. 8t+7, so an aligned 64-k block is held
// by 8 neighbouring lanes.  Optionally writes the row's compute-dtype copy;
// for 16-bit compute also its split v = hi + lo per 64-k block (hi = v rounded
// to the grid 2^(e-8), e = floor(log2 max|v|) of the block, the same split the
// contraction applies to x); returns {|v|_2, |lo|_2}.  A block whose grid
// exponent exceeds 100 cannot be split with the fp32 rounding constant: |lo|_2
// is then reported as +inf, which makes the contraction re-evaluate that row's
// elements in fp64.  With `vec` the source row is read, and the outputs
// written, 16 bytes at a time (rows start 16-byte aligned and K % 8 == 0).
// The stored and compute dtypes and `vec` are template arguments: with them
// as run-time values every element took the branches of all combinations.
template <int SRC_DT, int C_DT, bool VEC>
__device__ __forceinline__ void row_pass_t(const void* src, int64_t row, int64_t K, bool zero, void* dst, void* dst_hi,
                                           void* dst_lo, double2* norm_out) {
    constexpr int src_dt = SRC_DT, c_dt = C_DT;
    constexpr bool vec = VEC;
    __shared__ double red[2][4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    double ss = 0.0, ll = 0.0;
    bool wide = false;
    // RB chunks of 2048 values per round: a thread's loads of a round are
    // issued together (one memory round trip per 8192 values of the row)
    constexpr int RB = 4;
    for (int64_t kr = 0; kr < K; kr += 2048 * RB) {
        float cr[RB][8];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const int64_t kt = kr + 2048 * rb + 8 * tid;
            const bool in = kt < K;   // K % 8 == 0: a thread's 8 elements are all in or all out
            float* c = cr[rb];
            if (vec && in && !zero) {
                if (src_dt == DT_F32) {
                    const f32x4 a = *(const f32x4*)((const float*)src + row * K + kt);
                    const f32x4 b = *(const f32x4*)((const float*)src + row * K + kt + 4);
#pragma unroll
                    for (int i = 0; i < 4; ++i) { c[i] = a[i]; c[i + 4] = b[i]; }
                } else {
                    const i32x4 v = *(const i32x4*)((const uint16_t*)src + row * K + kt);
                    const i32x4 w = v;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint32_t u = (uint32_t)w[i];
                        c[2 * i] = src_dt == DT_F16 ? f16_to_f32((uint16_t)u) : bf16_to_f32((uint16_t)u);
                        c[2 * i + 1] = src_dt == DT_F16 ? f16_to_f32((uint16_t)(u >> 16)) : bf16_to_f32((uint16_t)(u >> 16));
                    }
                }
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) c[i] = (in && !zero) ? load_as_f32(src, src_dt, row * K + kt + i) : 0.f;
            }
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const int64_t kt = kr + 2048 * rb + 8 * tid;
            const bool in = kt < K;
            float* c = cr[rb];
            if (kr + 2048 * rb >= K) break;   // (uniform over the workgroup)
            // round to the compute dtype (exact when the stored dtype is the compute dtype)
            uint16_t h16[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                if (c_dt == DT_F16) { h16[i] = f32_to_f16(c[i]); c[i] = f16_to_f32(h16[i]); }
                else if (c_dt == DT_BF16) { h16[i] = f32_to_bf16(c[i]); c[i] = bf16_to_f32(h16[i]); }
            }
            if (dst && in) {
                if (c_dt == DT_F32) {
                    float* d = (float*)dst + row * K + kt;
                    if (vec) {
                        *(f32x4*)d = f32x4{c[0], c[1], c[2], c[3]};
                        *(f32x4*)(d + 4) = f32x4{c[4], c[5], c[6], c[7]};
                    } else {
#pragma unroll
                        for (int i = 0; i < 8; ++i) d[i] = c[i];
                    }
                } else {
                    *(i32x4*)((uint16_t*)dst + row * K + kt) =
                        i32x4{(int)(h16[0] | ((uint32_t)h16[1] << 16)), (int)(h16[2] | ((uint32_t)h16[3] << 16)),
                              (int)(h16[4] | ((uint32_t)h16[5] << 16)), (int)(h16[6] | ((uint32_t)h16[7] << 16))};
                }
            }
            float mx = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                ss = __builtin_fma((double)c[i], (double)c[i], ss);
                mx = __builtin_fmaxf(mx, __builtin_fabsf(c[i]));
            }
            if (dst_hi) {
                // maximum over the 64-k block: 8 lanes
#pragma unroll
                for (int o = 4; o >= 1; o >>= 1) mx = __builtin_fmaxf(mx, __shfl_xor(mx, o));
                int g = 0;
                float magic = 0.f;
                if (mx > 0.f) {
                    g = floor_log2(mx) - 8;
                    wide |= g > 100;
                    magic = __builtin_ldexpf(1.5f, (g > 100 ? 100 : g) + 23);
                }
                uint16_t hb[8], lb[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float hi = mx > 0.f ? (c[i] + magic) - magic : 0.f;
                    const float lo = c[i] - hi;
                    hb[i] = c_dt == DT_F16 ? f32_to_f16(hi) : f32_to_bf16(hi);
                    lb[i] = c_dt == DT_F16 ? f32_to_f16(lo) : f32_to_bf16(lo);
                    ll = __builtin_fma((double)lo, (double)lo, ll);
                }
                if (in) {
                    *(i32x4*)((uint16_t*)dst_hi + row * K + kt) =
                        i32x4{(int)(hb[0] | ((uint32_t)hb[1] << 16)), (int)(hb[2] | ((uint32_t)hb[3] << 16)),
                              (int)(hb[4] | ((uint32_t)hb[5] << 16)), (int)(hb[6] | ((uint32_t)hb[7] << 16))};
                    *(i32x4*)((uint16_t*)dst_lo + row * K + kt) =
                        i32x4{(int)(lb[0] | ((uint32_t)lb[1] << 16)), (int)(lb[2] | ((uint32_t)lb[3] << 16)),
                              (int)(lb[4] | ((uint32_t)lb[5] << 16)), (int)(lb[6] | ((uint32_t)lb[7] << 16))};
                }
            }
        }
    }
    // row sums: 64 lanes by shuffles, then the 4 waves through LDS
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        ss += __shfl_xor(ss, o);
        ll += __shfl_xor(ll, o);
    }
    if (lane == 0) {
        red[0][wave] = ss;
        red[1][wave] = ll;
    }
    __syncthreads();
    if (tid == 0) {
        const double s2 = (red[0][0] + red[0][1]) + (red[0][2] + red[0][3]);
        const double l2 = (red[1][0] + red[1][1]) + (red[1][2] + red[1][3]);
        *norm_out = double2{__builtin_sqrt(s2), wide ? __builtin_inf() : __builtin_sqrt(l2)};
    }
}

__device__ __forceinline__ void row_pass(const void* src, int src_dt, int c_dt, int64_t row, int64_t K, bool zero,
                                         bool vec, void* dst, void* dst_hi, void* dst_lo, double2* norm_out) {
#define LYC_ROW_PASS(S, C)                                                                             \
    if (src_dt == S && c_dt == C) {                                                                    \
        if (vec) row_pass_t<S, C, true>(src, row, K, zero, dst, dst_hi, dst_lo, norm_out);             \
        else row_pass_t<S, C, false>(src, row, K, zero, dst, dst_hi, dst_lo, norm_out);                \
        return;                                                                                        \
    }
    LYC_ROW_PASS(DT_F16, DT_F16)
    LYC_ROW_PASS(DT_BF16, DT_BF16)
    LYC_ROW_PASS(DT_F32, DT_F16)
    LYC_ROW_PASS(DT_F32, DT_BF16)
    LYC_ROW_PASS(DT_F32, DT_F32)
    LYC_ROW_PASS(DT_F16, DT_F32)
    LYC_ROW_PASS(DT_BF16, DT_F32)
    LYC_ROW_PASS(DT_F16, DT_BF16)
    LYC_ROW_PASS(DT_BF16, DT_F16)
#undef LYC_ROW_PASS
}

// fp32 -> 16-bit compute copy of elements [8 i0, 8 i1) and the tail past
// n8: 8 elements per thread and iteration, two 16-byte loads and one
// 16-byte store (src 16-byte aligned, dst 256-byte aligned)
__device__ __forceinline__ void cast_range(const float* __restrict__ src, uint16_t* __restrict__ dst, int64_t n,
                                           int c_dt, int64_t first, int64_t stride) {
    const int64_t n8 = n / 8;
    for (int64_t i = first; i < n8; i += stride) {
        const f32x4 a = ((const f32x4*)src)[2 * i];
        const f32x4 b = ((const f32x4*)src)[2 * i + 1];
        uint32_t o[4];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            o[e] = c_dt == DT_F16 ? pack_f16x2(a[2 * e], a[2 * e + 1]) : pack_bf16x2(a[2 * e], a[2 * e + 1]);
            o[2 + e] = c_dt == DT_F16 ? pack_f16x2(b[2 * e], b[2 * e + 1]) : pack_bf16x2(b[2 * e], b[2 * e + 1]);
        }
        ((i32x4*)dst)[i] = i32x4{(int)o[0], (int)o[1], (int)o[2], (int)o[3]};
    }
    for (int64_t i = n8 * 8 + first; i < n; i += stride)
        dst[i] = c_dt == DT_F16 ? f32_to_f16(src[i]) : f32_to_bf16(src[i]);
}

// blocks [0, r_pad): one row of down each (+ its split and norms); then up,
// grid-stride over up_blocks; then the fp32 operand casts (a2: x and W stored
// in fp32 under a 16-bit policy), grid-stride over the remaining blocks.  The
// row passes are latency-bound and the casts stream through HBM, so one
// launch runs both at once.
__global__ __launch_bounds__(256) void prep_kernel(PrepParams p) {
    const int b = blockIdx.x, tid = threadIdx.x;
    if (b == 0 && p.flagged != nullptr)
        for (int64_t i = tid; i < p.flag_slots; i += 256) p.flagged[i] = 0u;
    if (b >= p.r_pad + p.up_blocks) {
        const int64_t cb = b - (p.r_pad + p.up_blocks), nb = (int64_t)gridDim.x - (p.r_pad + p.up_blocks);
        for (int c = 0; c < 2; ++c)
            if (p.cast_n[c] > 0)
                cast_range(p.cast_src[c], (uint16_t*)p.cast_dst[c], p.cast_n[c], p.c_dt, cb * 256 + tid, nb * 256);
        return;
    }
    if (b < p.r_pad) {
        const bool split = p.c_dt != DT_F32;
        row_pass(p.down, p.down_dt, p.c_dt, b, p.K, b >= p.rank, p.vec, p.dc, split ? p.dh : nullptr,
                 split ? p.dl : nullptr, &p.dnorm[b]);
    } else {
        const int64_t total = p.N * (int64_t)p.r_pad;
        const int64_t stride = (int64_t)p.up_blocks * 256;
        for (int64_t i = (int64_t)(b - p.r_pad) * 256 + tid; i < total; i += stride) {
            const int64_t n = i / p.r_pad;
            const int j = (int)(i - n * p.r_pad);
            const float v = j < p.rank ? load_as_f32(p.up, p.up_dt, n * p.rank + j) : 0.f;
            double c;
            store_c(p.uc, i, v, p.c_dt, &c);
        }
    }
}

// split and norms of the rows of an operand already in the 16-bit compute
// dtype; clears *flagged
__global__ __launch_bounds__(256) void rownorm_kernel(const void* b, int c_dt, int64_t K, void* b_hi, void* b_lo,
                                                      double2* out, unsigned* flagged) {
    if (blockIdx.x == 0 && threadIdx.x == 0 && flagged) *flagged = 0u;
    row_pass(b, c_dt, c_dt, blockIdx.x, K, false, true, nullptr, b_hi, b_lo, &out[blockIdx.x]);
}

hipError_t launch_rownorm(const void* b, int c_dt, int64_t rows, int64_t K, void* b_hi, void* b_lo, double2* out,
                          unsigned* flagged, hipStream_t s) {
    hipLaunchKernelGGL(rownorm_kernel, dim3((unsigned)rows), dim3(256), 0, s, b, c_dt, K, b_hi, b_lo, out, flagged);
    return hipGetLastError();
}

hipError_t launch_prep(const PrepParams& p_in, hipStream_t s) {
    PrepParams p = p_in;
    // uc == nullptr: no up copy is wanted (the caller reads up as stored, or
    // not at all), so only the down rows are prepared
    const int64_t total = p.uc != nullptr ? p.N * (int64_t)p.r_pad : 0;
    int64_t up_blocks = (total + 255) / 256;
    if (up_blocks > 2048) up_blocks = 2048;
    if (up_blocks < 1 && p.uc != nullptr) up_blocks = 1;
    p.up_blocks = (int)up_blocks;
    // cast blocks: one 8-element chunk per thread up to 8192 blocks
    const int64_t cast8 = (p.cast_n[0] + p.cast_n[1]) / 8 + 1;
    int64_t cast_blocks = (p.cast_n[0] + p.cast_n[1]) > 0 ? (cast8 + 255) / 256 : 0;
    if (cast_blocks > 8192) cast_blocks = 8192;
    const int64_t blocks = p.r_pad + up_blocks + cast_blocks;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(prep_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p);
    return hipGetLastError();
}

// fp32 -> 16-bit compute copy on its own (the backward's casts)
__global__ __launch_bounds__(256) void cast_kernel(const float* __restrict__ src, uint16_t* __restrict__ dst,
                                                   int64_t n, int c_dt) {
    cast_range(src, dst, n, c_dt, (int64_t)blockIdx.x * 256 + threadIdx.x, (int64_t)gridDim.x * 256);
}

hipError_t launch_cast(const float* src, void* dst, int64_t n, int c_dt, hipStream_t s) {
    int64_t blocks = (n / 8 + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(cast_kernel, dim3((unsigned)blocks), dim3(256), 0, s, src, (uint16_t*)dst, n, c_dt);
    return hipGetLastError();
}

}  // namespace lyc
