// hpass.hip -- the low-rank contraction h = x_c . down_c^T and its rounding to
// the compute (storage) dtype, h_r = round_c(h) (LyCORIS "Precision" page,
// "Measured accuracy": the intermediate is rounded to the storage dtype before
// its second dot, as the eager two-Linear chain does).
//
// The rounding decision is taken on the exact h, not on an fp32 running sum:
// an fp32 sum that lands on the other side of a rounding midpoint than the
// exact value would move the whole output row by scale * ulp(h) * up.  So:
//   * each MFMA step (32 products for 16-bit compute) starts from zero and its
//     fp32 result is added into an fp64 accumulator;
//   * the error of that sum is bounded by  guard * 2^-24 * |x_m|_2 * |d_j|_2
//     (Cauchy-Schwarz bound on sum_k |x_mk d_jk|, times the per-step error
//     factor of the MFMA);
//   * when [h - E, h + E] straddles a rounding boundary of the 16-bit format,
//     the element is re-evaluated as an fp64 dot product over K (one wave per
//     element, products exact) before rounding.
// For fp32 compute the rounding to fp32 moves y by O(2^-24) and no guard is
// needed.
//
// Work split: a workgroup of 4 waves owns 64 rows; a wave owns 16 rows and all
// r_pad = 16*JB columns.  down_c is staged through LDS (shared by the 4 waves);
// each lane streams its own x fragment straight from HBM (x is read once).
#include "kernels.h"
#include "lyc_device.h"

namespace lyc {

template <class CT>
__device__ __forceinline__ float sumsq16(i32x4 v) {
    float s = 0.f;
    if (CT::dt == DT_F32) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float f = __builtin_bit_cast(float, v[i]);
            s += f * f;
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t u = (uint32_t)v[i];
            const float a = CT::dt == DT_F16 ? f16_to_f32((uint16_t)u) : bf16_to_f32((uint16_t)u);
            const float b = CT::dt == DT_F16 ? f16_to_f32((uint16_t)(u >> 16)) : bf16_to_f32((uint16_t)(u >> 16));
            s += a * a + b * b;
        }
    }
    return s;
}

// exact products of two 16-byte fragments, summed in fp64
template <class CT>
__device__ __forceinline__ double dot16_f64(i32x4 a, i32x4 b) {
    double s = 0.0;
    if (CT::dt == DT_F32) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            s = __builtin_fma((double)__builtin_bit_cast(float, a[i]), (double)__builtin_bit_cast(float, b[i]), s);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int hlf = 0; hlf < 2; ++hlf) {
                const uint16_t ua = (uint16_t)((uint32_t)a[i] >> (16 * hlf));
                const uint16_t ub = (uint16_t)((uint32_t)b[i] >> (16 * hlf));
                const double fa = CT::dt == DT_F16 ? (double)f16_to_f32(ua) : (double)bf16_to_f32(ua);
                const double fb = CT::dt == DT_F16 ? (double)f16_to_f32(ub) : (double)bf16_to_f32(ub);
                s = __builtin_fma(fa, fb, s);
            }
        }
    }
    return s;
}

template <class CT>
__device__ __forceinline__ uint16_t round16(double v) {
    return CT::dt == DT_F16 ? f64_to_f16(v) : f64_to_bf16(v);
}

template <class CT, int JB>
__global__ __launch_bounds__(256) void hpass_kernel(HpassParams p) {
    constexpr int RP = JB * 16;           // padded rank
    constexpr int DCH = RP * 8 / 256;     // 16-byte chunks of the down tile per thread
    __shared__ __attribute__((aligned(16))) char sd[2][RP * 128];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t wg_m0 = (int64_t)blockIdx.x * 64;
    const int rows_wg = (int)((p.M - wg_m0) < 64 ? (p.M - wg_m0) : 64);
    const uint32_t kbytes = (uint32_t)(p.K * CT::es);
    const int my_row = wave * 16 + (lane & 15);   // row within the workgroup
    const auto rsx = make_rsrc((const char*)p.x + wg_m0 * kbytes, (uint32_t)rows_wg * kbytes);
    const auto rsd = make_rsrc(p.d, (uint32_t)RP * kbytes);

    double acc[JB][4];
#pragma unroll
    for (int jb = 0; jb < JB; ++jb)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[jb][e] = 0.0;
    float sq = 0.f;

    const int KT = (int)((kbytes + 127) / 128);
    i32x4 dr[DCH], xr[2], xn[2];
    auto load_d = [&](uint32_t kb0) {
#pragma unroll
        for (int i = 0; i < DCH; ++i) {
            const int c = tid + i * 256;
            const uint32_t kb = kb0 + ((c & 7) << 4);
            dr[i] = buf_load16(rsd, kb < kbytes ? (uint32_t)(c >> 3) * kbytes + kb : OOB);
        }
    };
    auto store_d = [&](char* dst) {
#pragma unroll
        for (int i = 0; i < DCH; ++i) {
            const int c = tid + i * 256;
            *(i32x4*)(dst + lds_off(c >> 3, c & 7)) = dr[i];
        }
    };
    auto load_x = [&](i32x4 (&dst)[2], uint32_t kb0) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const uint32_t kb = kb0 + (uint32_t)((s * 4 + (lane >> 4)) << 4);
            dst[s] = buf_load16(rsx, kb < kbytes ? (uint32_t)my_row * kbytes + kb : OOB);
        }
    };

    if (KT > 0) {
        load_d(0);
        load_x(xr, 0);
        store_d(sd[0]);
        __syncthreads();
    }
    for (int kt = 0; kt < KT; ++kt) {
        const char* cur = sd[kt & 1];
        const bool more = kt + 1 < KT;
        if (more) {
            load_d((uint32_t)(kt + 1) * 128);
            load_x(xn, (uint32_t)(kt + 1) * 128);
        }
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            sq += sumsq16<CT>(xr[s]);
            const int kc = s * 4 + (lane >> 4);
#pragma unroll
            for (int jb = 0; jb < JB; ++jb) {
                const i32x4 df = *(const i32x4*)(cur + lds_off(jb * 16 + (lane & 15), kc));
                const f32x4 c = CT::step(df, xr[s], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[jb][e] += (double)c[e];
            }
        }
        if (more) {
            store_d(sd[(kt + 1) & 1]);
            xr[0] = xn[0];
            xr[1] = xn[1];
        }
        __syncthreads();
    }

    // |x_m|^2 for this lane's row: the four lane groups hold disjoint k ranges
    sq += __shfl_xor(sq, 16);
    sq += __shfl_xor(sq, 32);
    const int64_t m = wg_m0 + my_row;
    const bool row_ok = m < p.M;

    if (CT::dt != DT_F32) {
        // guard: flag elements whose error interval straddles a rounding boundary
        const double xnorm = (double)__builtin_sqrtf(sq) * (1.0 + 0x1p-8);
        unsigned nflag = 0;
#pragma unroll
        for (int jb = 0; jb < JB; ++jb) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = jb * 16 + 4 * (lane >> 4) + e;
                const double E = (p.guard * 0x1p-24 + 0x1p-37) * xnorm * p.dnorm[j] * (1.0 + 0x1p-20);
                const double h = acc[jb][e];
                const bool flag = row_ok && round16<CT>(h - E) != round16<CT>(h + E);
                uint64_t mask = __ballot(flag);
                nflag += (unsigned)__builtin_popcountll(mask);
                while (mask) {
                    const int L = __builtin_ctzll(mask);
                    mask &= mask - 1;
                    const int64_t mL = wg_m0 + wave * 16 + (L & 15);
                    const int jL = jb * 16 + 4 * (L >> 4) + e;
                    const i32x4* xrow = (const i32x4*)((const char*)p.x + mL * kbytes);
                    const i32x4* drow = (const i32x4*)((const char*)p.d + (int64_t)jL * kbytes);
                    double part = 0.0;
                    for (uint32_t c = lane; c < kbytes / 16; c += 64) part += dot16_f64<CT>(xrow[c], drow[c]);
#pragma unroll
                    for (int o = 32; o >= 1; o >>= 1) part += __shfl_xor(part, o);
                    if (lane == L) acc[jb][e] = part;
                }
            }
        }
        if (lane == 0 && nflag) atomicAdd(p.flagged, nflag);
    }

    if (row_ok) {
#pragma unroll
        for (int jb = 0; jb < JB; ++jb) {
            const int j0 = jb * 16 + 4 * (lane >> 4);
            if (CT::dt == DT_F32) {
                float* hp = (float*)p.h + m * p.r_pad + j0;
                *(f32x4*)hp = f32x4{(float)acc[jb][0], (float)acc[jb][1], (float)acc[jb][2], (float)acc[jb][3]};
            } else {
                uint16_t o[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = round16<CT>(acc[jb][e]);
                uint16_t* hp = (uint16_t*)p.h + m * p.r_pad + j0;
                *(i32x2*)hp = i32x2{(int)(o[0] | ((uint32_t)o[1] << 16)), (int)(o[2] | ((uint32_t)o[3] << 16))};
            }
        }
    }
}

template <class CT>
static hipError_t run_h(const HpassParams& p, hipStream_t s) {
    const dim3 grid((unsigned)((p.M + 63) / 64));
    switch (p.r_pad) {
    case 32: hipLaunchKernelGGL((hpass_kernel<CT, 2>), grid, dim3(256), 0, s, p); break;
    case 64: hipLaunchKernelGGL((hpass_kernel<CT, 4>), grid, dim3(256), 0, s, p); break;
    case 128: hipLaunchKernelGGL((hpass_kernel<CT, 8>), grid, dim3(256), 0, s, p); break;
    case 256: hipLaunchKernelGGL((hpass_kernel<CT, 16>), grid, dim3(256), 0, s, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_hpass(int c_dt, const HpassParams& p, hipStream_t s) {
    if (c_dt == DT_F16) return run_h<CF16>(p, s);
    if (c_dt == DT_BF16) return run_h<CBF16>(p, s);
    return run_h<CF32>(p, s);
}

}  // namespace lyc
