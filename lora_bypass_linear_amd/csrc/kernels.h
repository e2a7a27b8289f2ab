// kernels.h -- host-side launchers of the gfx950 kernels (internal to the
// library; the public surface is include/lyc.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lyc {

// Output tiles (rows of a x rows of b per workgroup); fp32 compute has 128x128
// and 64x64 only.
enum { GEMM_TILE_AUTO = -1, GEMM_TILE_256x256 = 0, GEMM_TILE_192x256 = 1, GEMM_TILE_128x128 = 2,
       GEMM_TILE_64x64 = 3 };

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
    int vec_store;     // 1: y rows allow 4-element vector stores
    // ksplit > 1: the main K steps of every tile are split over ksplit
    // workgroups (the fold goes with the first); each writes its fp32 sums to
    // partial [ksplit][M][N] and a second kernel adds them in split order,
    // adds the bias and rounds once
    int ksplit;
    float* partial;
    // y = round_out(post * acc + b): 1 in the forward; the scale of a weight
    // gradient whose product has no fold
    float post = 1.0f;
    // output tile: GEMM_TILE_AUTO (the analytic pick) or one of GEMM_TILE_*
    int tile = GEMM_TILE_AUTO;
    // per output feature n: y = round_out(gain[n] * acc + b) in place of post
    // (the DoRA forward's m_n / norm_n; nullptr: none)
    const float* gain = nullptr;
    // both operands stored with the contraction index as rows (16-bit
    // compute, no fold): ta and tb together, a [K][lda_t] and b [K][ldb_t].
    // Each such matrix must stay below 1 GiB (one buffer range covers it).
    int ta = 0, tb = 0;
    int64_t lda_t = 0, ldb_t = 0;
    // 1: few token rows (M <= 32, tile left to the analytic pick, no gain):
    // one workgroup per 16 output features over all of K (gemm_skinny says
    // whether the launch takes it; ksplit and partial are then unused)
    int skinny = 0;
};

struct GemmCand {
    int tile, ksplit;
    double cost;   // the model's estimate, microseconds
};
// The planner's shortlist for an M x N x K product (+ rf fold steps), best
// first: the analytic pick (the tile and K split launch_gemm takes by
// itself), then the other tile / K-split pairs by modelled time.  Returns
// the number written (at most max_out, at most 7).
int gemm_plan(int64_t M, int64_t N, int64_t K, int64_t rf, int c_dt, GemmCand* out, int max_out);
// the largest K split among every candidate the planner may shortlist for
// this shape, whatever the device rates order them by (the workspace is
// sized for it)
int gemm_plan_ksplit_max(int64_t M, int64_t N, int64_t K, int c_dt);
void gemm_tile_dims(int tile, int* tn, int* tm);
// tile (written to *tile) and K split of a 16-bit contraction over the tokens
// read in place (M x N output, one side the rank, K tokens)
int gemm_tok_plan(int64_t M, int64_t N, int64_t K, int* tile);

// The planner's device model: CU count of the current device and its dense
// MFMA rates (16-bit and fp32 operands, flop/s) and HBM rate (bytes/s).  Until
// measured on the device, the rates are MI355X's published per-CU peaks
// scaled by the CU count (measured = 0); without a device, 256 CUs.
struct DeviceRates {
    int64_t cus;
    double mfma16, mfma32, hbm;
    int measured;
};
DeviceRates device_rates();
// times a 256 MiB device-to-device copy and MFMA loops on the device of
// stream s (blocking; 512 MiB allocated for the copy meanwhile) and keeps the
// rates for that device
hipError_t measure_device_rates(hipStream_t s);

// Exact-rounding contraction (h pass and plain affine projection):
// C = x_c . b^T with fp64-folded MFMA steps, a rounding guard and in-kernel
// fp64 re-evaluation of the guarded elements, then either h_r = round_c(C) or
// y = round_out(round_out(C) + b).
enum { XR_H = 0, XR_AFFINE = 1 };
struct XrParams {
    const void* x;          // [M,K] compute dtype
    const void* b;          // [Nc,K] compute dtype: b_hi (16-bit h pass), else b itself
    const void* b_lo;       // [Nc,K] b - b_hi (16-bit h pass)
    const void* b_full;     // [Nc,K] b (down_c or W_c), for the fp64 re-evaluation
    const double2* bnorm;   // [Nc] {|b_j|_2, |b_lo,j|_2} (16-bit h pass)
    int64_t M, Nc, K;
    int guard;              // 1: apply the rounding guard (16-bit rounding target)
    // count of re-evaluated elements: h pass, one counter (zeroed beforehand);
    // with flag_per_wg (and where the kernel splits b itself), one per
    // workgroup (flag_slots of them, each written by its workgroup with a
    // plain store, nothing cleared beforehand; their sum is the count)
    unsigned* flagged;
    int64_t flag_slots = 0;
    int flag_per_wg = 0;
    int mode;               // XR_H or XR_AFFINE
    void* out;              // h [M][ld_out] (compute dtype) or y [M][ld_out] (out_dt)
    int64_t ld_out;
    int out_dt;             // XR_AFFINE
    const void* bias;       // XR_AFFINE, nullptr: none
    int bias_dt;
    int vec_store;          // XR_AFFINE: rows allow 4-element vector stores
    double scale;           // XR_H: the value rounded is scale * C (1 in the forward)
    // XR_H, 16-bit compute, Nc = 16: b = down as stored, split in the kernel
    // and its norms taken there (b_lo and bnorm unused); the guard's count is
    // then written per workgroup (flag_slots of them)
    int split_b = 0;
};

// h for few token rows, one wave per element: h[m][j] (j < r_pad; 0 from
// rank on) = round_c of the fp64 dot of x_m and down_j, both [.,K] in the
// compute dtype with row stride K; the per-workgroup counts of elements that
// took the compensated re-summation go to flagged[workgroup].
struct HdotParams {
    const void* x;       // [M][K]
    const void* down;    // [rank][K] (rows >= rank never read)
    int64_t M, K, rank;
    int r_pad;
    int vec;             // rows 16-byte aligned and K * es a multiple of 16: 16-byte loads
    void* out;           // h [M][r_pad]
    unsigned* flagged;   // [hdot_workgroups(M, r_pad)]
};
int64_t hdot_workgroups(int64_t M, int64_t r_pad);
hipError_t launch_hdot(int c_dt, const HdotParams& p, hipStream_t s);

// Compute-dtype copies of down [rank,K] -> [r_pad,K] (+ its hi/lo split per
// 64-k block and row norms) and up [N,rank] -> [N,r_pad]; zero padding;
// clears *flagged (if not null); and the fp32 operand casts, in one launch.
struct PrepParams {
    const void* down;
    int down_dt;
    const void* up;
    int up_dt;
    void* dc;
    void* dh;   // hi part of down_c (16-bit compute), else unused
    void* dl;   // lo part
    void* uc;
    double2* dnorm;   // {|down_c,j|, |lo_j|}
    int vec;          // down rows start 16-byte aligned: vector loads
    unsigned* flagged;        // guard counts, all flag_slots of them cleared
    int64_t flag_slots = 1;
    int64_t N, K, rank;
    int r_pad;
    int c_dt;
    // fp32 operands narrowed to the 16-bit compute dtype in the same launch
    // (cast_n[i] == 0: none); dst 256-byte aligned
    const float* cast_src[2] = {nullptr, nullptr};
    void* cast_dst[2] = {nullptr, nullptr};
    int64_t cast_n[2] = {0, 0};
    int up_blocks = 0;   // set by launch_prep
};

hipError_t launch_gemm(int c_dt, const GemmParams& p, hipStream_t s);
bool gemm_skinny(int c_dt, const GemmParams& p);
// K splits launch_gemm uses for this shape (1: none; the partial sums then
// need ksplit * M * N * 4 bytes of workspace)
int gemm_ksplit(int64_t M, int64_t N, int64_t K, int c_dt);
// the output tile launch_gemm uses for this shape
void gemm_tile_shape(int64_t M, int64_t N, int c_dt, int* tn, int* tm);
hipError_t launch_xr(int c_dt, const XrParams& p, hipStream_t s);
// workgroups of the plain affine form's launch under 16-bit compute (its
// guard-count slots)
int64_t xr_affine_workgroups(int64_t M, int64_t N);
// workgroups of the plain affine contraction when W is split beforehand (its
// guard-count slots)
int64_t xr_affine_split_pass_workgroups(int64_t M, int64_t N);
// workgroups of the h pass that splits b in the kernel (XrParams::split_b;
// its guard-count slots); 0 where that form does not apply (Nc != 16)
int64_t xr_h_split_b_workgroups(int64_t M, int64_t Nc);
// hi/lo split (per 64-k block) of each row of b [rows,K] (16-bit compute
// dtype) and {|b_j|_2, |b_lo,j|_2}; also clears *flagged (if not null)
hipError_t launch_rownorm(const void* b, int c_dt, int64_t rows, int64_t K, void* b_hi, void* b_lo, double2* out,
                          unsigned* flagged, hipStream_t s);
hipError_t launch_prep(const PrepParams& p, hipStream_t s);
// fp32 [n] -> 16-bit compute dtype [n], round to nearest even
hipError_t launch_cast(const float* src, void* dst, int64_t n, int c_dt, hipStream_t s);

}  // namespace lyc
