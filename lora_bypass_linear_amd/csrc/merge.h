// merge.h -- host-side launchers of the LoRA merge kernels (internal to the
// library; the public surface is include/lyc.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lyc {

// The merge's operands: down^T_c [K][r_pad] and up_c [N][r_pad] in the
// compute dtype, the rank padded with zeros.
struct MergePrepParams {
    const void* down;
    int down_dt;
    const void* up;
    int up_dt;
    void* dt_c;
    void* uc;
    int64_t N, K, rank;
    int r_pad;
    int c_dt;
};
hipError_t launch_merge_prep(const MergePrepParams& p, hipStream_t s);

// W' = round_out(fma(scale, up_c . down_c, W)) per 128 x 128 tile of W [N][K]
struct MergeParams {
    const void* w;
    int w_dt;
    const void* dt_c;   // down^T_c [K][r_pad], compute dtype
    const void* uc;     // up_c [N][r_pad]
    void* out;          // W' [N][K] (may be w itself)
    int out_dt;
    int64_t N, K;
    int r_pad;          // 0: no bypass (W' = round_out(W))
    float scale;
    int vec;            // K a multiple of the lane chunk (8 elements when W and W' are 16-bit, else 4)
                        // and W, W' aligned to one chunk: 16-byte (8-byte for 16-bit W under fp32 W') accesses
    // DoRA row norms instead of W' (norm_partial != nullptr): per-tile sums of
    // squares [K tiles][N] fp32, then norms[n] = sqrt of their sum in tile order
    float* norm_partial = nullptr;
    float* norms = nullptr;
    // down [rank][K] and up [N][rank] read as stored, in place of dt_c and uc
    // (16-bit compute, both already in it, rank and K multiples of 8, 16-byte
    // aligned, rank * K * 2 below 2^31); nullptr: the prepared copies
    const void* down_raw = nullptr;
    const void* up_raw = nullptr;
    int64_t rank = 0;
};
hipError_t launch_merge(int c_dt, const MergeParams& p, hipStream_t s);
// whether launch_merge takes the streaming form for these parameters (16-bit
// compute, W and W' in it, down and up read as stored, K a multiple of 8)
bool merge_streams(int c_dt, const MergeParams& p);
// after launch_merge in the norm mode: norms[n] = sqrt(sum of the partials, in order)
hipError_t launch_norm_finish(int c_dt, const MergeParams& p, hipStream_t s);
// gain[n] = m[n] / norms[n] in fp32 (the DoRA forward's per-feature factor)
hipError_t launch_dora_gain(const void* m, int m_dt, const float* norms, int64_t N, float* gain, hipStream_t s);

}  // namespace lyc
