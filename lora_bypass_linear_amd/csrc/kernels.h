// kernels.h -- host-side launchers of the gfx950 kernels (internal to the
// library; the public surface is include/lyc.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lyc {

// y = epilogue( [scale * (af . bf^T)] + a . b^T ) for one output tile per
// workgroup.  a = W_c [N,K], b = x_c [M,K], af = up_c [N,rf], bf = h_r [M,rf],
// all in the compute dtype, rows 16-byte aligned.
struct GemmParams {
    const void* a;
    const void* b;
    const void* af;   // nullptr when rf == 0
    const void* bf;
    int64_t M, N, K, rf;
    float scale;
    const void* bias;  // nullptr: no bias
    int bias_dt;
    void* y;
    int y_dt;
    int double_round;  // 1: y = round(round(acc) + b)  (plain affine contract)
    int vec_store;     // 1: y rows allow 4-element vector stores
};

// h_r = round_c(x_c . d_c^T), the guard and its fp64 re-evaluation.
struct HpassParams {
    const void* x;        // [M,K] compute dtype
    const void* d;        // [r_pad,K] compute dtype (rows >= rank are zero)
    const double* dnorm;  // [r_pad] Euclidean norms of the rows of d
    void* h;              // [M,r_pad] compute dtype
    int64_t M, K;
    int r_pad;
    double guard;         // error bound factor (units of 2^-24 * |x_m| * |d_j|)
    unsigned* flagged;    // count of re-evaluated elements
};

// Compute-dtype copies of down [rank,K] -> [r_pad,K] (+ row norms) and
// up [N,rank] -> [N,r_pad]; zero padding; clears *flagged.
struct PrepParams {
    const void* down;
    int down_dt;
    const void* up;
    int up_dt;
    void* dc;
    void* uc;
    double* dnorm;
    unsigned* flagged;
    int64_t N, K, rank;
    int r_pad;
    int c_dt;
};

hipError_t launch_gemm(int c_dt, const GemmParams& p, hipStream_t s);
// the output tile launch_gemm uses for this shape
void gemm_tile_shape(int64_t M, int64_t N, int c_dt, int* tn, int* tm);
hipError_t launch_hpass(int c_dt, const HpassParams& p, hipStream_t s);
hipError_t launch_prep(const PrepParams& p, hipStream_t s);
// fp32 [n] -> 16-bit compute dtype [n], round to nearest even
hipError_t launch_cast(const float* src, void* dst, int64_t n, int c_dt, hipStream_t s);

}  // namespace lyc
