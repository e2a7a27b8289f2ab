// api.cpp -- the C ABI (include/lyc.h): argument checks, the dtype policy,
// the workspace layout and the launch sequence.  Every check happens before
// the first launch, so a failed call has queued nothing.
#include "../../include/lyc.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <string>
#include <mutex>
#include <vector>

#include "bwd.h"
#include "kernels.h"
#include "merge.h"
#include "tune.h"

namespace {

constexpr int64_t MAX_RANK = 256;
constexpr int64_t MAX_DIM = (int64_t)1 << 30;
constexpr int64_t MAX_K = (int64_t)1 << 20;  // keeps per-tile byte offsets below 2^31

bool valid_dt(int dt) { return dt == LYC_F16 || dt == LYC_BF16 || dt == LYC_F32; }
size_t esize(int dt) { return dt == LYC_F32 ? 4 : 2; }
size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Dtype policy (LyCORIS "Precision" page, "Dtype policy").
int resolve(const int* dts, int n, int* compute, int* output) {
    if (dts == nullptr || n < 1) return LYC_ERR_INVALID_ARG;
    bool h16 = false, hbf = false, h32 = false;
    for (int i = 0; i < n; ++i) {
        switch (dts[i]) {
        case LYC_F16: h16 = true; break;
        case LYC_BF16: hbf = true; break;
        case LYC_F32: h32 = true; break;
        default: return LYC_ERR_INVALID_ARG;
        }
    }
    if (h16 && hbf) return LYC_ERR_MIXED_HALF;
    const int c = h16 ? LYC_F16 : (hbf ? LYC_BF16 : LYC_F32);
    if (compute) *compute = c;
    if (output) *output = h32 ? LYC_F32 : c;
    return LYC_OK;
}

struct Problem {
    bool lora;
    int64_t M, N, K, rank;
    int x_dt, w_dt, b_dt, d_dt, u_dt;
    int c_dt, o_dt;
    int r_pad;
    int m_dt = 0;    // DoRA: the magnitude vector's dtype (a policy operand); 0 otherwise
    bool w_kept = false;   // the caller passes W already rounded to the compute dtype
    // plain affine form: the workspace already holds W's compute-dtype copy
    // (fp32 W) and its split and row norms, from lyc_linear_prepare or an
    // earlier forward with the same W, shapes and dtypes
    bool w_prepared = false;
};

// Shape and dtype checks shared by the size queries and the forward calls.
int check_problem(Problem& P) {
    if (P.M < 0 || P.N < 0 || P.K < 0 || P.rank < 0) return LYC_ERR_INVALID_ARG;
    if (!valid_dt(P.x_dt) || !valid_dt(P.w_dt)) return LYC_ERR_INVALID_ARG;
    if (P.b_dt != 0 && !valid_dt(P.b_dt)) return LYC_ERR_INVALID_ARG;
    int dts[6], n = 0;
    dts[n++] = P.x_dt;
    dts[n++] = P.w_dt;
    if (P.b_dt != 0) dts[n++] = P.b_dt;
    if (P.lora) {
        if (!valid_dt(P.d_dt) || !valid_dt(P.u_dt)) return LYC_ERR_INVALID_ARG;
        dts[n++] = P.d_dt;
        dts[n++] = P.u_dt;
    }
    if (P.m_dt != 0) {
        if (!P.lora || !valid_dt(P.m_dt)) return LYC_ERR_INVALID_ARG;
        dts[n++] = P.m_dt;
    }
    const int st = resolve(dts, n, &P.c_dt, &P.o_dt);
    if (st != LYC_OK) return st;
    if (P.M > MAX_DIM || P.N > MAX_DIM || P.K > MAX_K) return LYC_ERR_UNSUPPORTED;
    if (P.K % 8 != 0) return LYC_ERR_UNSUPPORTED;
    if (P.rank > MAX_RANK) return LYC_ERR_UNSUPPORTED;
    if (!P.lora) P.rank = 0;
    P.r_pad = P.rank == 0 ? 0 : (P.rank <= 16 && P.c_dt != LYC_F32) ? 16 : (P.rank <= 32 ? 32 : P.rank <= 64 ? 64 : P.rank <= 128 ? 128 : 256);
    return LYC_OK;
}

struct Layout {
    size_t xc = 0, wc = 0, dc = 0, dh = 0, dl = 0, uc = 0, h = 0, dnorm = 0, wh = 0, wl = 0, wnorm = 0, flagged = 0,
           partial = 0, gain = 0, total = 0;
    // plain affine form: guard counts, one per workgroup of the contraction
    int64_t flag_slots = 0;
    bool w_split_pass = false;
    int ksplit = 1, ks_max = 1;
    bool cast_x = false, cast_w = false;
};

// h for few token rows: one wave per element (fp64 dots), in place of the
// split contraction, whose single workgroup would walk all of K
bool hdot_path(const Problem& P) {
    return P.lora && P.r_pad > 0 && P.K > 0 && P.M <= 128 && (double)P.M * (double)P.r_pad * (double)P.K <= 33554432.0;
}

// rank 16 with down already in the compute dtype: the split contraction
// splits down itself (no preparation pass; its guard counts per workgroup)
bool h_split_b_shape(const Problem& P) {
    return P.lora && !hdot_path(P) && P.c_dt != LYC_F32 && P.rank == 16 && P.r_pad == 16 && P.d_dt == P.c_dt &&
           P.M > 0 && P.K > 0;
}

Layout layout(const Problem& P) {
    Layout L;
    size_t off = 0;
    const size_t ce = esize(P.c_dt);
    L.cast_x = P.x_dt == LYC_F32 && P.c_dt != LYC_F32;
    L.cast_w = P.w_dt == LYC_F32 && P.c_dt != LYC_F32 && !P.w_kept;
    if (L.cast_x) { L.xc = off; off = align256(off + (size_t)(P.M * P.K) * 2); }
    const bool split = P.c_dt != LYC_F32;   // hi/lo split of the second contraction operand
    if (P.r_pad > 0) {
        L.dc = off; off = align256(off + (size_t)P.r_pad * (size_t)P.K * ce);
        if (split) {
            L.dh = off; off = align256(off + (size_t)P.r_pad * (size_t)P.K * ce);
            L.dl = off; off = align256(off + (size_t)P.r_pad * (size_t)P.K * ce);
        }
        L.uc = off; off = align256(off + (size_t)P.N * (size_t)P.r_pad * ce);
        L.h = off; off = align256(off + (size_t)P.M * (size_t)P.r_pad * ce);
        L.dnorm = off; off = align256(off + (size_t)P.r_pad * 2 * sizeof(double));
        // the guard's count: one counter, or one per workgroup of the few-row h
        // kernel or of the h pass that splits down itself
        L.flag_slots = hdot_path(P)         ? lyc::hdot_workgroups(P.M, P.r_pad)
                       : h_split_b_shape(P) ? lyc::xr_h_split_b_workgroups(P.M, P.r_pad)
                                            : 1;
        L.flagged = off; off = align256(off + (size_t)L.flag_slots * sizeof(unsigned));
    }
    if (P.lora) {
        // fp32 partial sums of a K-split GEMM (few output tiles), sized for
        // the largest split the planner can shortlist (a tuned pick may take it)
        L.ksplit = lyc::gemm_ksplit(P.M, P.N, P.K, P.c_dt);
        const int ks_max = lyc::gemm_plan_ksplit_max(P.M, P.N, P.K, P.c_dt);
        L.ks_max = ks_max;
        if (ks_max > 1) { L.partial = off; off = align256(off + (size_t)ks_max * (size_t)(P.M * P.N) * 4); }
        // DoRA: the per-feature gain m / norm in fp32
        if (P.m_dt != 0) { L.gain = off; off = align256(off + (size_t)P.N * 4); }
    }
    if (!P.lora && split) {
        // the projection's rounding guard: W's hi/lo split and row norms from the
        // row-norm pass and one counter, or, where the contraction splits W
        // itself, one count per workgroup
        const int64_t wgs = lyc::xr_affine_workgroups(P.M, P.N);
        L.w_split_pass = wgs == 0;
        if (L.w_split_pass) {
            L.wh = off; off = align256(off + (size_t)P.N * (size_t)P.K * ce);
            L.wl = off; off = align256(off + (size_t)P.N * (size_t)P.K * ce);
            L.wnorm = off; off = align256(off + (size_t)P.N * 2 * sizeof(double));
        }
        L.flag_slots = L.w_split_pass ? lyc::xr_affine_split_pass_workgroups(P.M, P.N) : wgs;
        L.flagged = off; off = align256(off + (size_t)L.flag_slots * sizeof(unsigned));
    }
    // the compute-dtype copy of an fp32 W last: a caller that keeps that copy
    // (lyc_lora_linear_fwd_wc) needs the same workspace without it, every
    // other region at the same offset
    if (L.cast_w) { L.wc = off; off = align256(off + (size_t)(P.N * P.K) * 2); }
    L.total = off;
    return L;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    if (a == nullptr || b == nullptr || na == 0 || nb == 0) return false;
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + nb && b0 < a0 + na;
}

// ---- optional per-kernel timing (lyc_profile_begin / lyc_profile_end) -------
struct ProfSlot {
    hipEvent_t a, b;
    int kind;
};
std::mutex g_prof_mu;
std::vector<ProfSlot> g_prof;   // created events
size_t g_prof_used = 0;
bool g_prof_on = false;

// Launch through `fn`, bracketed by an event pair when profiling is on.
template <class F>
hipError_t timed(int kind, hipStream_t s, F fn) {
    ProfSlot* slot = nullptr;
    {
        std::lock_guard<std::mutex> lk(g_prof_mu);
        if (g_prof_on && g_prof_used < g_prof.size()) {
            slot = &g_prof[g_prof_used++];
            slot->kind = kind;
        }
    }
    if (slot && hipEventRecord(slot->a, s) != hipSuccess) return hipErrorUnknown;
    const hipError_t e = fn();
    if (slot && hipEventRecord(slot->b, s) != hipSuccess) return hipErrorUnknown;
    return e;
}

// The GEMM configuration a LoRA forward runs with: `force` (while tuning),
// else a measured pick for this device and shape, else the analytic one.
int forward(const Problem& P, const void* x, const void* w, const void* bias, const void* down, const void* up,
            double scale, void* y, int y_dt, void* ws, size_t ws_bytes, void* stream,
            const lyc::TuneChoice* force = nullptr, const void* mag = nullptr, const float* norms = nullptr) {
    // (P.w_kept: w is W_c, W already rounded to the compute dtype)
    if (y_dt != P.o_dt) return LYC_ERR_DTYPE_MISMATCH;
    if ((bias == nullptr) != (P.b_dt == 0)) return LYC_ERR_INVALID_ARG;
    if (P.M == 0 || P.N == 0) return LYC_OK;
    if (y == nullptr) return LYC_ERR_INVALID_ARG;
    if (P.K > 0) {
        if (x == nullptr || w == nullptr) return LYC_ERR_INVALID_ARG;
        if (!aligned(x, 16) || !aligned(w, 16)) return LYC_ERR_UNSUPPORTED;
    }
    if (P.w_kept && P.K > 0 && overlaps(y, (size_t)(P.M * P.N) * esize(y_dt), w, (size_t)(P.N * P.K) * esize(P.c_dt)))
        return LYC_ERR_INVALID_ARG;
    if (P.rank > 0) {
        if (up == nullptr || (P.K > 0 && down == nullptr)) return LYC_ERR_INVALID_ARG;
        if (!aligned(up, esize(P.u_dt)) || !aligned(down, esize(P.d_dt))) return LYC_ERR_UNSUPPORTED;
    }
    if (bias && !aligned(bias, esize(P.b_dt))) return LYC_ERR_UNSUPPORTED;
    if (!aligned(y, esize(y_dt))) return LYC_ERR_UNSUPPORTED;
    const Layout L = layout(P);
    if (L.total > 0) {
        if (ws == nullptr || ws_bytes < L.total || !aligned(ws, 256)) return LYC_ERR_WORKSPACE;
    }
    hipStream_t s = (hipStream_t)stream;
    char* W = (char*)ws;
    (void)hipGetLastError();  // clear a stale error so the checks below see only ours

    const void* xa = x;
    const void* wa = w;
    const bool cx = L.cast_x && P.K > 0, cw = L.cast_w && P.K > 0;
    if (cx) xa = W + L.xc;
    if (cw) wa = W + L.wc;

    if (!P.lora) {
        if (cx && timed(LYC_KERNEL_CAST, s, [&] {
                return lyc::launch_cast((const float*)x, W + L.xc, P.M * P.K, P.c_dt, s);
            }) != hipSuccess)
            return LYC_ERR_HIP;
        if (cw && !P.w_prepared && timed(LYC_KERNEL_CAST, s, [&] {
                return lyc::launch_cast((const float*)w, W + L.wc, P.N * P.K, P.c_dt, s);
            }) != hipSuccess)
            return LYC_ERR_HIP;
        // plain affine: exact-rounding contraction with the round-then-add-bias
        // epilogue; W's split and row norms from the row-norm pass (skipped
        // when the workspace already holds them) or inside the contraction;
        // one guard count per workgroup, nothing to clear
        const bool guard = P.c_dt != LYC_F32 && y_dt != LYC_F32;
        if (L.w_split_pass && !P.w_prepared && timed(LYC_KERNEL_PREP, s, [&] {
                return lyc::launch_rownorm(wa, P.c_dt, P.N, P.K, W + L.wh, W + L.wl, (double2*)(W + L.wnorm),
                                           nullptr, s);
            }) != hipSuccess)
            return LYC_ERR_HIP;
        lyc::XrParams xp{};
        xp.x = xa;
        xp.b = L.w_split_pass ? (const void*)(W + L.wh) : wa;
        xp.b_lo = L.w_split_pass ? (const void*)(W + L.wl) : nullptr;
        xp.b_full = wa;
        xp.bnorm = L.w_split_pass ? (const double2*)(W + L.wnorm) : nullptr;
        xp.M = P.M;
        xp.Nc = P.N;
        xp.K = P.K;
        xp.guard = guard ? 1 : 0;
        xp.flagged = L.flag_slots > 0 ? (unsigned*)(W + L.flagged) : nullptr;
        xp.flag_slots = L.flag_slots;
        xp.flag_per_wg = 1;
        xp.mode = lyc::XR_AFFINE;
        xp.out = y;
        xp.ld_out = P.N;
        xp.out_dt = y_dt;
        xp.bias = bias;
        xp.bias_dt = P.b_dt;
        xp.vec_store = (P.N % 4 == 0) && aligned(y, y_dt == LYC_F32 ? 16 : 8);
        xp.scale = 1.0;
        if (timed(LYC_KERNEL_GEMM, s, [&] { return lyc::launch_xr(P.c_dt, xp, s); }) != hipSuccess) return LYC_ERR_HIP;
        return LYC_OK;
    }

    lyc::GemmParams g{};
    g.a = wa;
    g.b = xa;
    g.M = P.M;
    g.N = P.N;
    g.K = P.K;
    g.bias = bias;
    g.bias_dt = P.b_dt;
    g.y = y;
    g.y_dt = y_dt;
    g.scale = (float)scale;
    g.rf = 0;
    g.ksplit = L.ksplit;
    g.post = 1.0f;
    lyc::TuneChoice tc{};
    const bool have = force ? (tc = *force, true)
                            : lyc::tune_count() > 0 &&
                                  lyc::tune_lookup(lyc::tune_key("lora_fwd", P.M, P.N, P.K, P.r_pad, P.c_dt, P.o_dt), &tc);
    // a pick is taken only if this build can run it in this workspace
    if (have && tc.ksplit >= 1 && tc.ksplit <= L.ks_max && tc.tile >= 0 && tc.tile <= 3 &&
        (P.c_dt != LYC_F32 || tc.tile == lyc::GEMM_TILE_128x128 || tc.tile == lyc::GEMM_TILE_64x64)) {
        g.tile = tc.tile;
        g.ksplit = tc.ksplit;
    }
    g.partial = g.ksplit > 1 ? (float*)(W + L.partial) : nullptr;
    // few token rows, no stored pick: one workgroup per 16 output features
    // over all of K (no K split, no second kernel)
    g.skinny = P.M <= 32 ? 1 : 0;
    if (P.m_dt != 0) {
        float* gain = (float*)(W + L.gain);
        if (timed(LYC_KERNEL_PREP, s, [&] { return lyc::launch_dora_gain(mag, P.m_dt, norms, P.N, gain, s); }) !=
            hipSuccess)
            return LYC_ERR_HIP;
        g.gain = gain;
    }
    const uintptr_t vec_align = y_dt == LYC_F32 ? 16 : 8;
    g.vec_store = (P.N % 4 == 0) && aligned(y, vec_align);

    // up already in the compute dtype, unpadded (rank == r_pad) and 16-byte
    // aligned: the fold reads it as stored and the prep makes no copy
    const bool up_stored = P.r_pad > 0 && P.u_dt == P.c_dt && P.rank == P.r_pad && aligned(up, 16);
    // few token rows, or rank 16, with the factors already in the compute
    // dtype: no preparation of them (h reads down as stored, the fold reads
    // up as stored)
    const bool hdot = hdot_path(P);
    const bool hsb = h_split_b_shape(P) && aligned(down, 16);
    const bool factors = P.r_pad > 0 && !((hdot || hsb) && up_stored && P.d_dt == P.c_dt);
    if (factors || cx || cw) {
        // one launch: the factors' preparation and the fp32 operand casts
        lyc::PrepParams pp{};
        if (factors) {
            pp.down = down;
            pp.down_dt = P.d_dt;
            pp.up = up;
            pp.up_dt = P.u_dt;
            pp.dc = W + L.dc;
            pp.dh = W + L.dh;
            pp.dl = W + L.dl;
            pp.uc = up_stored ? nullptr : W + L.uc;
            pp.dnorm = (double2*)(W + L.dnorm);
            // (where the workspace has a count per workgroup of a form this
            // call does not take, every slot is cleared: their sum is the count)
            pp.flagged = (unsigned*)(W + L.flagged);
            pp.flag_slots = L.flag_slots;
            pp.vec = aligned(down, 16) ? 1 : 0;
        }
        pp.N = P.N;
        pp.K = P.K;
        pp.rank = P.rank;
        pp.r_pad = factors ? P.r_pad : 0;
        pp.c_dt = P.c_dt;
        int nc = 0;
        if (cx) { pp.cast_src[nc] = (const float*)x; pp.cast_dst[nc] = W + L.xc; pp.cast_n[nc++] = P.M * P.K; }
        if (cw) { pp.cast_src[nc] = (const float*)w; pp.cast_dst[nc] = W + L.wc; pp.cast_n[nc++] = P.N * P.K; }
        if (timed(LYC_KERNEL_PREP, s, [&] { return lyc::launch_prep(pp, s); }) != hipSuccess) return LYC_ERR_HIP;
    }
    if (P.r_pad > 0 && hdot) {
        lyc::HdotParams hq{};
        hq.x = xa;
        hq.down = P.d_dt == P.c_dt ? down : (const void*)(W + L.dc);
        hq.M = P.M;
        hq.K = P.K;
        hq.rank = P.rank;
        hq.r_pad = P.r_pad;
        hq.vec = ((P.K * (int64_t)esize(P.c_dt)) % 16 == 0 && aligned(xa, 16) && aligned(hq.down, 16)) ? 1 : 0;
        hq.out = W + L.h;
        hq.flagged = (unsigned*)(W + L.flagged);
        if (timed(LYC_KERNEL_HPASS, s, [&] { return lyc::launch_hdot(P.c_dt, hq, s); }) != hipSuccess)
            return LYC_ERR_HIP;
        g.af = up_stored ? up : (const void*)(W + L.uc);
        g.bf = W + L.h;
        g.rf = P.r_pad;
    } else if (P.r_pad > 0) {
        lyc::XrParams hp{};
        const bool split = P.c_dt != LYC_F32;
        hp.x = xa;
        if (hsb) {
            hp.b = down;
            hp.b_full = down;
            hp.split_b = 1;
            hp.flag_slots = L.flag_slots;
        } else {
            hp.b = W + (split ? L.dh : L.dc);
            hp.b_lo = split ? (const void*)(W + L.dl) : nullptr;
            hp.b_full = W + L.dc;
            hp.bnorm = (const double2*)(W + L.dnorm);
        }
        hp.M = P.M;
        hp.Nc = P.r_pad;
        hp.K = P.K;
        hp.guard = P.c_dt != LYC_F32 ? 1 : 0;
        hp.flagged = (unsigned*)(W + L.flagged);
        hp.mode = lyc::XR_H;
        hp.out = W + L.h;
        hp.ld_out = P.r_pad;
        hp.scale = 1.0;
        if (timed(LYC_KERNEL_HPASS, s, [&] { return lyc::launch_xr(P.c_dt, hp, s); }) != hipSuccess)
            return LYC_ERR_HIP;

        g.af = up_stored ? up : (const void*)(W + L.uc);
        g.bf = W + L.h;
        g.rf = P.r_pad;
    }
    if (timed(LYC_KERNEL_GEMM, s, [&] { return lyc::launch_gemm(P.c_dt, g, s); }) != hipSuccess) return LYC_ERR_HIP;
    return LYC_OK;
}

// ---- LoRA merge: W' = round_out(W + scale * up_c . down_c) ------------------
struct Merge {
    int64_t N, K, rank;
    int w_dt, d_dt, u_dt;
    int c_dt, o_dt;
    int r_pad;
    size_t dt_c, uc, total;   // workspace: down^T_c [K][r_pad], up_c [N][r_pad]
};

int check_merge(Merge& G) {
    if (G.N < 0 || G.K < 0 || G.rank < 0) return LYC_ERR_INVALID_ARG;
    if (!valid_dt(G.w_dt) || !valid_dt(G.d_dt) || !valid_dt(G.u_dt)) return LYC_ERR_INVALID_ARG;
    const int dts[3] = {G.w_dt, G.d_dt, G.u_dt};
    const int st = resolve(dts, 3, &G.c_dt, &G.o_dt);
    if (st != LYC_OK) return st;
    if (G.N > MAX_DIM || G.K > MAX_DIM || G.N * G.K > ((int64_t)1 << 38)) return LYC_ERR_UNSUPPORTED;
    if (G.rank > MAX_RANK) return LYC_ERR_UNSUPPORTED;
    G.r_pad = G.rank == 0 ? 0 : G.rank <= 16 ? 16 : G.rank <= 32 ? 32 : G.rank <= 64 ? 64 : G.rank <= 128 ? 128 : 256;
    const size_t ce = esize(G.c_dt);
    size_t off = 0;
    G.dt_c = off; off = align256(off + (size_t)G.K * (size_t)G.r_pad * ce);
    G.uc = off; off = align256(off + (size_t)G.N * (size_t)G.r_pad * ce);
    G.total = G.r_pad > 0 ? off : 0;
    return LYC_OK;
}

// down and up can be read as stored (no preparation pass): both already in a
// 16-bit compute dtype, rank and K multiples of 8 (16-byte chunks), 16-byte
// aligned, and down below 2 GiB (one buffer range).  Rank rows past the rank
// (up to the next multiple of 64) are read through offsets past the range,
// which return zero; those rows too must lie below 2 GiB, or their 32-bit
// offsets could wrap back into down.
bool merge_reads_as_stored(const Merge& G, const void* down, const void* up) {
    return G.rank > 0 && G.c_dt != LYC_F32 && G.d_dt == G.c_dt && G.u_dt == G.c_dt && G.rank % 8 == 0 &&
           G.K % 8 == 0 && aligned(down, 16) && aligned(up, 16) &&
           ((G.rank + 63) / 64) * 64 * G.K * 2 < ((int64_t)1 << 31);
}

// The factors' preparation pass (down^T_c and up_c), unless both are read as stored
int merge_prepare(const Merge& G, const void* down, const void* up, bool raw, char* W, hipStream_t s) {
    if (G.r_pad == 0 || raw) return LYC_OK;
    lyc::MergePrepParams mp{};
    mp.down = down;
    mp.down_dt = G.d_dt;
    mp.up = up;
    mp.up_dt = G.u_dt;
    mp.dt_c = W + G.dt_c;
    mp.uc = W + G.uc;
    mp.N = G.N;
    mp.K = G.K;
    mp.rank = G.rank;
    mp.r_pad = G.r_pad;
    mp.c_dt = G.c_dt;
    return timed(LYC_KERNEL_PREP, s, [&] { return lyc::launch_merge_prep(mp, s); }) == hipSuccess ? LYC_OK
                                                                                               : LYC_ERR_HIP;
}

int merge(const Merge& G, const void* w, const void* down, const void* up, double scale, void* out, int out_dt,
          void* ws, size_t ws_bytes, void* stream) {
    if (out_dt != G.o_dt) return LYC_ERR_DTYPE_MISMATCH;
    if (!(scale == scale) || scale > 3.4e38 || scale < -3.4e38) return LYC_ERR_INVALID_ARG;
    if (G.N == 0 || G.K == 0) return LYC_OK;
    if (w == nullptr || out == nullptr) return LYC_ERR_INVALID_ARG;
    if (G.rank > 0 && (down == nullptr || up == nullptr)) return LYC_ERR_INVALID_ARG;
    // out may be w itself (each element's W is read before it is written),
    // but no other overlap
    const uintptr_t wb = (uintptr_t)w, we = wb + (uintptr_t)(G.N * G.K) * esize(G.w_dt);
    const uintptr_t ob = (uintptr_t)out, oe = ob + (uintptr_t)(G.N * G.K) * esize(out_dt);
    if (ob != wb && ob < we && wb < oe) return LYC_ERR_INVALID_ARG;
    if (ob == wb && G.w_dt != out_dt) return LYC_ERR_INVALID_ARG;
    if (!aligned(w, esize(G.w_dt)) || !aligned(out, esize(out_dt))) return LYC_ERR_UNSUPPORTED;
    if (G.rank > 0 && (!aligned(down, esize(G.d_dt)) || !aligned(up, esize(G.u_dt)))) return LYC_ERR_UNSUPPORTED;
    if (G.total > 0 && (ws == nullptr || ws_bytes < G.total || !aligned(ws, 256))) return LYC_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    char* W = (char*)ws;
    (void)hipGetLastError();
    const bool raw = merge_reads_as_stored(G, down, up);
    lyc::MergeParams mg{};
    mg.w = w;
    mg.w_dt = G.w_dt;
    mg.dt_c = W + G.dt_c;
    mg.uc = W + G.uc;
    mg.out = out;
    mg.out_dt = out_dt;
    mg.N = G.N;
    mg.K = G.K;
    mg.r_pad = G.r_pad;
    mg.scale = (float)scale;
    // 8 elements per lane chunk when W and W' are both 16-bit, else 4
    const int E = (G.w_dt == LYC_F32 || out_dt == LYC_F32) ? 4 : 8;
    mg.vec = (G.K % E == 0) && aligned(w, E * esize(G.w_dt)) && aligned(out, E * esize(out_dt));
    if (raw) {
        mg.down_raw = down;
        mg.up_raw = up;
        mg.rank = G.rank;
    }
    if (merge_prepare(G, down, up, raw, W, s) != LYC_OK) return LYC_ERR_HIP;
    if (timed(LYC_KERNEL_GEMM, s, [&] { return lyc::launch_merge(G.c_dt, mg, s); }) != hipSuccess) return LYC_ERR_HIP;
    return LYC_OK;
}

// ---- LoRA-bypass backward ------------------------------------------------------
// BWD_WT: the caller passes W_c^T; BWD_H: the caller passes the forward's h_r
enum { BWD_DX = 1, BWD_DDOWN = 2, BWD_DUP = 4, BWD_WT = 8, BWD_H = 16 };

struct Bwd {
    Problem P;       // the forward's problem; c_dt resolved over (x, W, b, down, up, dy)
    int dy_dt;
    int want;        // BWD_* bits
    int64_t M8;      // tokens rounded up to 8: row length of the transposed token-major copies
};

struct BwdLayout {
    size_t xc = 0, gc = 0, dc = 0, dh = 0, dl = 0, uc = 0, dnorm = 0, flag_h = 0, h = 0, ut = 0, uth = 0, utl = 0,
           unorm = 0, flag_g = 0, gh = 0, wt = 0, dt = 0, xt = 0, ght = 0, dyt = 0, ht = 0, partial = 0, total = 0;
    bool cast_x = false, cast_g = false, need_h = false, need_gh = false;
    // tr_tok: dDown and dUp read x, dy, h_r and gh_r as stored, the token
    // index as their contraction rows (16-bit compute, each operand below
    // 1 GiB); else they read transposed copies.  dx reads W^T and down^T copies.
    bool tr_tok = false;
    int ks_dx = 1, ks_dd = 1, ks_du = 1;
    int tile_dd = lyc::GEMM_TILE_AUTO, tile_du = lyc::GEMM_TILE_AUTO;   // tr_tok: lyc::gemm_tok_plan's tiles
};

int check_bwd(Bwd& B) {
    Problem& P = B.P;
    if (P.M < 0 || P.N < 0 || P.K < 0 || P.rank < 0 || B.want < 0 || B.want > 31) return LYC_ERR_INVALID_ARG;
    if (!valid_dt(P.x_dt) || !valid_dt(P.w_dt) || !valid_dt(P.d_dt) || !valid_dt(P.u_dt) || !valid_dt(B.dy_dt))
        return LYC_ERR_INVALID_ARG;
    if (P.b_dt != 0 && !valid_dt(P.b_dt)) return LYC_ERR_INVALID_ARG;
    int dts[6], n = 0;
    dts[n++] = P.x_dt;
    dts[n++] = P.w_dt;
    if (P.b_dt != 0) dts[n++] = P.b_dt;
    dts[n++] = P.d_dt;
    dts[n++] = P.u_dt;
    dts[n++] = B.dy_dt;
    const int st = resolve(dts, n, &P.c_dt, &P.o_dt);
    if (st != LYC_OK) return st;
    // every dimension is the contraction length of one of the products (M of
    // dDown and dUp, N of dx and gh, K of h): the limit of K in the forward
    if (P.M > MAX_K || P.N > MAX_K || P.K > MAX_K) return LYC_ERR_UNSUPPORTED;
    if (P.K % 8 != 0 || P.N % 8 != 0) return LYC_ERR_UNSUPPORTED;
    if (P.rank > MAX_RANK) return LYC_ERR_UNSUPPORTED;
    P.r_pad = P.rank == 0 ? 0 : (P.rank <= 16 && P.c_dt != LYC_F32) ? 16 : (P.rank <= 32 ? 32 : P.rank <= 64 ? 64 : P.rank <= 128 ? 128 : 256);
    B.M8 = (P.M + 7) & ~(int64_t)7;
    return LYC_OK;
}

BwdLayout bwd_layout(const Bwd& B) {
    const Problem& P = B.P;
    BwdLayout L;
    size_t off = 0;
    const size_t ce = esize(P.c_dt);
    const bool split = P.c_dt != LYC_F32;
    const bool dx = B.want & BWD_DX, dd = (B.want & BWD_DDOWN) && P.rank > 0, du = (B.want & BWD_DUP) && P.rank > 0;
    L.need_h = du && !(B.want & BWD_H);     // h_r feeds dUp only (recomputed unless the caller passes it)
    L.need_gh = P.rank > 0 && (dx || dd);   // gh_r feeds dx's fold and dDown
    const size_t G1 = (size_t)1 << 30;
    L.tr_tok = split && (size_t)P.M * (size_t)P.K * 2 < G1 && (size_t)P.M * (size_t)P.N * 2 < G1;
    L.cast_x = P.x_dt == LYC_F32 && P.c_dt != LYC_F32 && (L.need_h || (L.tr_tok && dd));
    L.cast_g = B.dy_dt == LYC_F32 && P.c_dt != LYC_F32 && (L.need_gh || dx || (L.tr_tok && du));
    auto take = [&](size_t& at, size_t bytes) { at = off; off = align256(off + bytes); };
    const size_t M = (size_t)P.M, N = (size_t)P.N, K = (size_t)P.K, R = (size_t)P.r_pad, M8 = (size_t)B.M8;
    if (L.cast_x) take(L.xc, M * K * 2);
    if (L.cast_g) take(L.gc, M * N * 2);
    if (L.need_h) {
        take(L.dc, R * K * ce);
        if (split) { take(L.dh, R * K * ce); take(L.dl, R * K * ce); }
        take(L.dnorm, R * 2 * sizeof(double));
        take(L.flag_h, sizeof(unsigned));
        take(L.h, M * R * ce);
    }
    if (L.need_gh) {
        take(L.ut, R * N * ce);
        if (split) { take(L.uth, R * N * ce); take(L.utl, R * N * ce); }
        take(L.unorm, R * 2 * sizeof(double));
        take(L.flag_g, sizeof(unsigned));
        take(L.gh, M * R * ce);
    }
    size_t part = 0;
    const int64_t Kt = L.tr_tok ? P.M : B.M8;   // contraction length of the token GEMMs
    if (dx) {
        if (!(B.want & BWD_WT)) take(L.wt, K * N * ce);
        if (P.rank > 0) take(L.dt, K * R * ce);
        L.ks_dx = lyc::gemm_ksplit(P.M, P.K, P.N, P.c_dt);
        if (L.ks_dx > 1) part = std::max(part, (size_t)L.ks_dx * M * K * 4);
    }
    if (dd) {
        if (!L.tr_tok) {
            take(L.xt, K * M8 * ce);
            take(L.ght, R * M8 * ce);
        }
        L.ks_dd = L.tr_tok ? lyc::gemm_tok_plan(P.rank, P.K, Kt, &L.tile_dd) : lyc::gemm_ksplit(P.rank, P.K, Kt, P.c_dt);
        if (L.ks_dd > 1) part = std::max(part, (size_t)L.ks_dd * (size_t)P.rank * K * 4);
    }
    if (du) {
        if (!L.tr_tok) {
            take(L.dyt, N * M8 * ce);
            take(L.ht, R * M8 * ce);
        }
        L.ks_du = L.tr_tok ? lyc::gemm_tok_plan(P.N, P.rank, Kt, &L.tile_du) : lyc::gemm_ksplit(P.N, P.rank, Kt, P.c_dt);
        if (L.ks_du > 1) part = std::max(part, (size_t)L.ks_du * N * (size_t)P.rank * 4);
    }
    if (part > 0) take(L.partial, part);
    L.total = off;
    return L;
}

int backward(const Bwd& B, const void* x, const void* w, const void* down, const void* up, double scale,
             const void* dy, void* dx, void* d_down, void* d_up, void* ws, size_t ws_bytes, void* stream,
             const void* w_t = nullptr, const void* h_r = nullptr) {
    const Problem& P = B.P;
    if (!(scale == scale) || scale > 3.4e38 || scale < -3.4e38) return LYC_ERR_INVALID_ARG;
    const bool wdx = B.want & BWD_DX, wdd = B.want & BWD_DDOWN, wdu = B.want & BWD_DUP;
    const bool wt_given = B.want & BWD_WT;
    const int64_t M = P.M, N = P.N, K = P.K, r = P.rank;
    // which inputs the wanted gradients read
    const bool use_x = (wdd || wdu) && r > 0 && M > 0 && K > 0;
    const bool use_dy = M > 0 && N > 0 && (wdx || r > 0);
    const bool use_w = wdx && M > 0 && N > 0 && K > 0;
    const bool use_f = r > 0 && M > 0;
    if ((use_x && x == nullptr) || (use_dy && dy == nullptr) || (use_w && (wt_given ? w_t : w) == nullptr) ||
        (use_f && (down == nullptr || up == nullptr)))
        return LYC_ERR_INVALID_ARG;
    // a caller-kept W_c^T [K][N] is read in place by the dx GEMM: 16-byte rows
    if (wt_given && use_w && !aligned(w_t, 16)) return LYC_ERR_UNSUPPORTED;
    // the forward's h_r [M][r_pad], read in place by dUp (16-byte rows)
    const bool h_given = B.want & BWD_H;
    const bool use_h = h_given && wdu && r > 0 && M > 0 && N > 0;
    if (use_h && h_r == nullptr) return LYC_ERR_INVALID_ARG;
    if (use_h && !aligned(h_r, 16)) return LYC_ERR_UNSUPPORTED;
    const size_t ndx = (size_t)(M * K) * esize(P.x_dt), ndd = (size_t)(r * K) * esize(P.d_dt),
                 ndu = (size_t)(N * r) * esize(P.u_dt);
    if ((wdx && ndx > 0 && dx == nullptr) || (wdd && ndd > 0 && d_down == nullptr) || (wdu && ndu > 0 && d_up == nullptr))
        return LYC_ERR_INVALID_ARG;
    // alignment: rows read in place by the contractions need 16 bytes
    const bool x_in_place = use_x && P.x_dt == P.c_dt, dy_in_place = use_dy && B.dy_dt == P.c_dt;
    if ((x_in_place && !aligned(x, 16)) || (dy_in_place && !aligned(dy, 16))) return LYC_ERR_UNSUPPORTED;
    if ((w && !aligned(w, esize(P.w_dt))) || (down && !aligned(down, esize(P.d_dt))) ||
        (up && !aligned(up, esize(P.u_dt))) || (x && !aligned(x, esize(P.x_dt))) ||
        (dy && !aligned(dy, esize(B.dy_dt))))
        return LYC_ERR_UNSUPPORTED;
    if ((wdx && dx && !aligned(dx, esize(P.x_dt))) || (wdd && d_down && !aligned(d_down, esize(P.d_dt))) ||
        (wdu && d_up && !aligned(d_up, esize(P.u_dt))))
        return LYC_ERR_UNSUPPORTED;
    // the gradients overlap neither the inputs nor each other
    const void* ins[7] = {x, w, down, up, dy, wt_given ? w_t : nullptr, use_h ? h_r : nullptr};
    const size_t nin[7] = {(size_t)(M * K) * esize(P.x_dt), (size_t)(N * K) * esize(P.w_dt),
                           (size_t)(r * K) * esize(P.d_dt), (size_t)(N * r) * esize(P.u_dt),
                           (size_t)(M * N) * esize(B.dy_dt), (size_t)(K * N) * esize(P.c_dt),
                           (size_t)(M * P.r_pad) * esize(P.c_dt)};
    void* outs[3] = {wdx ? dx : nullptr, wdd ? d_down : nullptr, wdu ? d_up : nullptr};
    const size_t nout[3] = {ndx, ndd, ndu};
    for (int i = 0; i < 3; ++i) {
        for (int j = 0; j < 7; ++j)
            if (overlaps(outs[i], nout[i], ins[j], nin[j])) return LYC_ERR_INVALID_ARG;
        for (int j = i + 1; j < 3; ++j)
            if (overlaps(outs[i], nout[i], outs[j], nout[j])) return LYC_ERR_INVALID_ARG;
    }
    const BwdLayout L = bwd_layout(B);
    if (L.total > 0 && (ws == nullptr || ws_bytes < L.total || !aligned(ws, 256))) return LYC_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    char* W = (char*)ws;
    (void)hipGetLastError();
    const bool split = P.c_dt != LYC_F32;
    auto transpose = [&](const void* src, int src_dt, int64_t rows, int64_t cols, void* dst, int64_t rows_pad,
                         int64_t cols_pad) {
        lyc::TransposeParams tp{src, src_dt, rows, cols, dst, P.c_dt, rows_pad, cols_pad};
        return timed(LYC_KERNEL_CAST, s, [&] { return lyc::launch_transpose(tp, s); }) == hipSuccess;
    };
    auto gemm = [&](lyc::GemmParams& g) {
        return timed(LYC_KERNEL_GEMM, s, [&] { return lyc::launch_gemm(P.c_dt, g, s); }) == hipSuccess;
    };

    // compute-dtype copies of fp32 operands that are read in place
    const void* xa = x;
    const void* ga = dy;
    if (L.cast_x && M * K > 0) {
        if (timed(LYC_KERNEL_CAST, s, [&] { return lyc::launch_cast((const float*)x, W + L.xc, M * K, P.c_dt, s); }) !=
            hipSuccess)
            return LYC_ERR_HIP;
        xa = W + L.xc;
    }
    if (L.cast_g && M * N > 0) {
        if (timed(LYC_KERNEL_CAST, s, [&] { return lyc::launch_cast((const float*)dy, W + L.gc, M * N, P.c_dt, s); }) !=
            hipSuccess)
            return LYC_ERR_HIP;
        ga = W + L.gc;
    }

    // h_r, recomputed exactly as the forward computes it (only dUp reads it)
    if (L.need_h && M > 0) {
        lyc::PrepParams pp{};
        pp.down = down;
        pp.down_dt = P.d_dt;
        pp.up = up;
        pp.up_dt = P.u_dt;
        pp.dc = W + L.dc;
        pp.dh = W + L.dh;
        pp.dl = W + L.dl;
        pp.uc = nullptr;   // the backward's products read up^T (gh) only
        pp.dnorm = (double2*)(W + L.dnorm);
        pp.flagged = (unsigned*)(W + L.flag_h);
        pp.N = N;
        pp.K = K;
        pp.rank = r;
        pp.r_pad = P.r_pad;
        pp.c_dt = P.c_dt;
        pp.vec = aligned(down, 16) ? 1 : 0;
        if (timed(LYC_KERNEL_PREP, s, [&] { return lyc::launch_prep(pp, s); }) != hipSuccess) return LYC_ERR_HIP;
        lyc::XrParams hp{};
        hp.x = xa;
        hp.b = W + (split ? L.dh : L.dc);
        hp.b_lo = split ? (const void*)(W + L.dl) : nullptr;
        hp.b_full = W + L.dc;
        hp.bnorm = (const double2*)(W + L.dnorm);
        hp.M = M;
        hp.Nc = P.r_pad;
        hp.K = K;
        hp.guard = split ? 1 : 0;
        hp.flagged = (unsigned*)(W + L.flag_h);
        hp.mode = lyc::XR_H;
        hp.out = W + L.h;
        hp.ld_out = P.r_pad;
        hp.scale = 1.0;
        if (timed(LYC_KERNEL_HPASS, s, [&] { return lyc::launch_xr(P.c_dt, hp, s); }) != hipSuccess) return LYC_ERR_HIP;
    }

    // gh_r = round_c(scale * dy_c . up_c): the h pass over dy with b = up_c^T
    if (L.need_gh && M > 0 && N == 0) {
        // no outputs: gh = 0 (a transpose of an empty source writes only its zero padding)
        if (!transpose(W, P.c_dt, 0, 0, W + L.gh, P.r_pad, M)) return LYC_ERR_HIP;
    } else if (L.need_gh && M > 0) {
        if (!transpose(up, P.u_dt, N, r, W + L.ut, N, P.r_pad)) return LYC_ERR_HIP;
        if (split && timed(LYC_KERNEL_PREP, s, [&] {
                return lyc::launch_rownorm(W + L.ut, P.c_dt, P.r_pad, N, W + L.uth, W + L.utl,
                                           (double2*)(W + L.unorm), (unsigned*)(W + L.flag_g), s);
            }) != hipSuccess)
            return LYC_ERR_HIP;
        lyc::XrParams gp{};
        gp.x = ga;
        gp.b = W + (split ? L.uth : L.ut);
        gp.b_lo = split ? (const void*)(W + L.utl) : nullptr;
        gp.b_full = W + L.ut;
        gp.bnorm = (const double2*)(W + L.unorm);
        gp.M = M;
        gp.Nc = P.r_pad;
        gp.K = N;
        gp.guard = split ? 1 : 0;
        gp.flagged = (unsigned*)(W + L.flag_g);
        gp.mode = lyc::XR_H;
        gp.out = W + L.gh;
        gp.ld_out = P.r_pad;
        gp.scale = scale;
        if (timed(LYC_KERNEL_HPASS, s, [&] { return lyc::launch_xr(P.c_dt, gp, s); }) != hipSuccess) return LYC_ERR_HIP;
    }

    // dx = round_x(dy_c . W_c + gh_r . down_c): the forward's GEMM with W^T, the fold over down^T
    if (wdx && M > 0 && K > 0) {
        lyc::GemmParams g{};
        if (!wt_given && N > 0 && !transpose(w, P.w_dt, N, K, W + L.wt, N, K)) return LYC_ERR_HIP;
        if (r > 0 && !transpose(down, P.d_dt, r, K, W + L.dt, P.r_pad, K)) return LYC_ERR_HIP;
        g.a = wt_given ? w_t : (const void*)(W + L.wt);
        g.af = r > 0 ? (const void*)(W + L.dt) : nullptr;
        g.b = ga;
        g.M = M;
        g.N = K;
        g.K = N;
        g.bf = r > 0 ? (const void*)(W + L.gh) : nullptr;
        g.rf = r > 0 ? P.r_pad : 0;
        g.scale = 1.0f;
        g.post = 1.0f;
        g.y = dx;
        g.y_dt = P.x_dt;
        g.ksplit = L.ks_dx;
        g.partial = L.ks_dx > 1 ? (float*)(W + L.partial) : nullptr;
        g.vec_store = (K % 4 == 0) && aligned(dx, P.x_dt == LYC_F32 ? 16 : 8);
        if (!gemm(g)) return LYC_ERR_HIP;
    }

    // dDown = round_down(gh_r^T . x_c), over the tokens
    if (wdd && r > 0 && K > 0) {
        lyc::GemmParams g{};
        if (L.tr_tok) {
            // x_c [M][K] and gh_r [M][r_pad] as stored: tokens are their rows
            g.a = M > 0 ? xa : W;
            g.b = W + L.gh;
            g.ta = g.tb = 1;
            g.lda_t = K;
            g.ldb_t = P.r_pad;
            g.K = M;
        } else {
            if (M > 0) {
                if (!transpose(x, P.x_dt, M, K, W + L.xt, B.M8, K)) return LYC_ERR_HIP;
                if (!transpose(W + L.gh, P.c_dt, M, P.r_pad, W + L.ght, B.M8, P.r_pad)) return LYC_ERR_HIP;
            }
            g.a = W + L.xt;
            g.b = W + L.ght;
            g.K = B.M8;
        }
        g.M = r;
        g.N = K;
        g.rf = 0;
        g.scale = 1.0f;
        g.post = 1.0f;
        g.y = d_down;
        g.y_dt = P.d_dt;
        g.tile = L.tile_dd;
        g.ksplit = L.ks_dd;
        g.partial = L.ks_dd > 1 ? (float*)(W + L.partial) : nullptr;
        g.vec_store = (K % 4 == 0) && aligned(d_down, P.d_dt == LYC_F32 ? 16 : 8);
        if (!gemm(g)) return LYC_ERR_HIP;
    }

    // dUp = round_up(scale * dy_c^T . h_r), over the tokens
    if (wdu && r > 0 && N > 0) {
        lyc::GemmParams g{};
        const void* hs = use_h ? h_r : (const void*)(W + L.h);
        if (L.tr_tok) {
            // h_r [M][r_pad] and dy_c [M][N] as stored: tokens are their rows
            g.a = hs;
            g.b = M > 0 ? ga : W;
            g.ta = g.tb = 1;
            g.lda_t = P.r_pad;
            g.ldb_t = N;
            g.K = M;
        } else {
            if (M > 0) {
                if (!transpose(dy, B.dy_dt, M, N, W + L.dyt, B.M8, N)) return LYC_ERR_HIP;
                if (!transpose(hs, P.c_dt, M, P.r_pad, W + L.ht, B.M8, P.r_pad)) return LYC_ERR_HIP;
            }
            g.a = W + L.ht;
            g.b = W + L.dyt;
            g.K = B.M8;
        }
        g.M = N;
        g.N = r;
        g.rf = 0;
        g.scale = 1.0f;
        g.post = (float)scale;
        g.y = d_up;
        g.y_dt = P.u_dt;
        g.tile = L.tile_du;
        g.ksplit = L.ks_du;
        g.partial = L.ks_du > 1 ? (float*)(W + L.partial) : nullptr;
        g.vec_store = (r % 4 == 0) && aligned(d_up, P.u_dt == LYC_F32 ? 16 : 8);
        if (!gemm(g)) return LYC_ERR_HIP;
    }
    return LYC_OK;
}

}  // namespace

extern "C" {

int lyc_gemm_plan(int64_t M, int64_t N, int64_t K, int64_t rf, int compute_dt, int max_out, int* count, int* tile_n,
                  int* tile_m, int* ksplit, double* cost_us) {
    if (M < 0 || N < 0 || K < 0 || rf < 0 || !valid_dt(compute_dt) || max_out < 0) return LYC_ERR_INVALID_ARG;
    lyc::GemmCand c[8];
    const int n = lyc::gemm_plan(M, N, K, rf, compute_dt, c, max_out < 8 ? max_out : 8);
    if (count) *count = n;
    for (int i = 0; i < n; ++i) {
        int tn, tm;
        lyc::gemm_tile_dims(c[i].tile, &tn, &tm);
        if (tile_n) tile_n[i] = tn;
        if (tile_m) tile_m[i] = tm;
        if (ksplit) ksplit[i] = c[i].ksplit;
        if (cost_us) cost_us[i] = c[i].cost;
    }
    return LYC_OK;
}

int lyc_device_rates(int64_t* cus, double* mfma16_flops, double* mfma32_flops, double* hbm_bytes_per_s,
                     int* measured) {
    const lyc::DeviceRates r = lyc::device_rates();
    if (cus) *cus = r.cus;
    if (mfma16_flops) *mfma16_flops = r.mfma16;
    if (mfma32_flops) *mfma32_flops = r.mfma32;
    if (hbm_bytes_per_s) *hbm_bytes_per_s = r.hbm;
    if (measured) *measured = r.measured;
    return LYC_OK;
}

int lyc_measure_device_rates(void* stream) {
    return lyc::measure_device_rates((hipStream_t)stream) == hipSuccess ? LYC_OK : LYC_ERR_HIP;
}

int lyc_lora_linear_tune(const void* x, int x_dt, const void* w, int w_dt, const void* bias, int bias_dt,
                         const void* down, int down_dt, const void* up, int up_dt, int64_t rank, double scale,
                         void* y, int y_dt, int64_t M, int64_t N, int64_t K, void* workspace, size_t workspace_bytes,
                         void* stream, int* tile_n, int* tile_m, int* ksplit, double* best_ms, double* cand_ms) {
    Problem P{true, M, N, K, rank, x_dt, w_dt, bias_dt, down_dt, up_dt, 0, 0, 0};
    int st = check_problem(P);
    if (st != LYC_OK) return st;
    if (!valid_dt(y_dt)) return LYC_ERR_INVALID_ARG;
    if (!(scale == scale) || scale > 3.4e38 || scale < -3.4e38) return LYC_ERR_INVALID_ARG;
    const std::string key = lyc::tune_key("lora_fwd", M, N, K, P.r_pad, P.c_dt, P.o_dt);
    if (key.empty()) return LYC_ERR_HIP;
    const char* env = std::getenv("LYC_KERNEL_TUNE");
    const bool timing = !(env && (std::strcmp(env, "off") == 0 || std::strcmp(env, "0") == 0));
    // the shortlist is ordered by this device's measured rates
    if (timing && !lyc::device_rates().measured && lyc::measure_device_rates((hipStream_t)stream) != hipSuccess)
        return LYC_ERR_HIP;
    lyc::GemmCand plan[8];
    const int np = lyc::gemm_plan(M, N, K, P.r_pad, P.c_dt, plan, 7);
    lyc::TuneChoice best{plan[0].tile, plan[0].ksplit, 0.0};
    if (timing && M > 0 && N > 0) {
        hipStream_t s = (hipStream_t)stream;
        hipEvent_t a, b;
        if (hipEventCreate(&a) != hipSuccess) return LYC_ERR_HIP;
        if (hipEventCreate(&b) != hipSuccess) { (void)hipEventDestroy(a); return LYC_ERR_HIP; }
        double best_t = 1e300;
        for (int i = 0; i < np && st == LYC_OK; ++i) {
            const lyc::TuneChoice c{plan[i].tile, plan[i].ksplit, 0.0};
            st = forward(P, x, w, bias, down, up, scale, y, y_dt, workspace, workspace_bytes, stream, &c);   // warm
            double t_min = 1e300;
            for (int rep = 0; rep < 3 && st == LYC_OK; ++rep) {
                float ms = 0.f;
                if (hipEventRecord(a, s) != hipSuccess) { st = LYC_ERR_HIP; break; }
                st = forward(P, x, w, bias, down, up, scale, y, y_dt, workspace, workspace_bytes, stream, &c);
                if (st != LYC_OK) break;
                if (hipEventRecord(b, s) != hipSuccess || hipEventSynchronize(b) != hipSuccess ||
                    hipEventElapsedTime(&ms, a, b) != hipSuccess) { st = LYC_ERR_HIP; break; }
                t_min = std::min(t_min, (double)ms);
            }
            if (cand_ms) cand_ms[i] = t_min;
            if (st == LYC_OK && t_min < best_t) { best_t = t_min; best = c; best.ms = t_min; }
        }
        (void)hipEventDestroy(a);
        (void)hipEventDestroy(b);
        if (st != LYC_OK) return st;
    }
    lyc::tune_store(key, best);
    int tn, tm;
    lyc::gemm_tile_dims(best.tile, &tn, &tm);
    if (tile_n) *tile_n = tn;
    if (tile_m) *tile_m = tm;
    if (ksplit) *ksplit = best.ksplit;
    if (best_ms) *best_ms = best.ms;
    return LYC_OK;
}

int lyc_tuning_key(int64_t M, int64_t N, int64_t K, int64_t rank, int x_dt, int w_dt, int bias_dt, int down_dt,
                   int up_dt, char* buf, size_t len) {
    Problem P{true, M, N, K, rank, x_dt, w_dt, bias_dt, down_dt, up_dt, 0, 0, 0};
    const int st = check_problem(P);
    if (st != LYC_OK) return st;
    const std::string key = lyc::tune_key("lora_fwd", M, N, K, P.r_pad, P.c_dt, P.o_dt);
    if (key.empty()) return LYC_ERR_HIP;
    if (buf == nullptr || len < key.size() + 1) return LYC_ERR_INVALID_ARG;
    std::memcpy(buf, key.c_str(), key.size() + 1);
    return LYC_OK;
}

int lyc_tuning_lookup(int64_t M, int64_t N, int64_t K, int64_t rank, int x_dt, int w_dt, int bias_dt, int down_dt,
                      int up_dt, int* found, int* tile_n, int* tile_m, int* ksplit) {
    Problem P{true, M, N, K, rank, x_dt, w_dt, bias_dt, down_dt, up_dt, 0, 0, 0};
    const int st = check_problem(P);
    if (st != LYC_OK) return st;
    lyc::TuneChoice c{};
    const bool f = lyc::tune_lookup(lyc::tune_key("lora_fwd", M, N, K, P.r_pad, P.c_dt, P.o_dt), &c);
    if (found) *found = f ? 1 : 0;
    if (f) {
        int tn, tm;
        lyc::gemm_tile_dims(c.tile, &tn, &tm);
        if (tile_n) *tile_n = tn;
        if (tile_m) *tile_m = tm;
        if (ksplit) *ksplit = c.ksplit;
    }
    return LYC_OK;
}

int lyc_tuning_save(const char* path) {
    if (path == nullptr) return LYC_ERR_INVALID_ARG;
    return lyc::tune_save(path) == 0 ? LYC_OK : LYC_ERR_IO;
}

int lyc_tuning_load(const char* path, int* entries) {
    if (path == nullptr) return LYC_ERR_INVALID_ARG;
    return lyc::tune_load(path, entries) == 0 ? LYC_OK : LYC_ERR_IO;
}

int lyc_tuning_clear(void) {
    lyc::tune_clear();
    return LYC_OK;
}

int lyc_tuning_count(void) { return lyc::tune_count(); }

int lyc_lora_linear_bwd_workspace_size(int64_t M, int64_t N, int64_t K, int64_t rank, int x_dt, int w_dt,
                                       int bias_dt, int down_dt, int up_dt, int dy_dt, int want, size_t* bytes) {
    Bwd B{Problem{true, M, N, K, rank, x_dt, w_dt, bias_dt, down_dt, up_dt, 0, 0, 0}, dy_dt, want, 0};
    const int st = check_bwd(B);
    if (st != LYC_OK) return st;
    if (bytes) *bytes = bwd_layout(B).total;
    return LYC_OK;
}

int lyc_lora_linear_bwd(const void* x, int x_dt, const void* w, int w_dt, int bias_dt, const void* down,
                        int down_dt, const void* up, int up_dt, int64_t rank, double scale, const void* dy,
                        int dy_dt, void* dx, void* d_down, void* d_up, int64_t M, int64_t N, int64_t K,
                        void* workspace, size_t workspace_bytes, void* stream) {
    const int want = (dx ? BWD_DX : 0) | (d_down ? BWD_DDOWN : 0) | (d_up ? BWD_DUP : 0);
    Bwd B{Problem{true, M, N, K, rank, x_dt, w_dt, bias_dt, down_dt, up_dt, 0, 0, 0}, dy_dt, want, 0};
    const int st = check_bwd(B);
    if (st != LYC_OK) return st;
    return backward(B, x, w, down, up, scale, dy, dx, d_down, d_up, workspace, workspace_bytes, stream);
}

int lyc_lora_linear_bwd_wt(const void* x, int x_dt, const void* w_t, int w_dt, int bias_dt, const void* down,
                           int down_dt, const void* up, int up_dt, int64_t rank, double scale, const void* dy,
                           int dy_dt, void* dx, void* d_down, void* d_up, int64_t M, int64_t N, int64_t K,
                           void* workspace, size_t workspace_bytes, void* stream) {
    const int want = (dx ? BWD_DX : 0) | (d_down ? BWD_DDOWN : 0) | (d_up ? BWD_DUP : 0) | BWD_WT;
    Bwd B{Problem{true, M, N, K, rank, x_dt, w_dt, bias_dt, down_dt, up_dt, 0, 0, 0}, dy_dt, want, 0};
    const int st = check_bwd(B);
    if (st != LYC_OK) return st;
    return backward(B, x, nullptr, down, up, scale, dy, dx, d_down, d_up, workspace, workspace_bytes, stream, w_t);
}

int lyc_lora_linear_bwd_saved(const void* x, int x_dt, const void* w, const void* w_t, int w_dt, int bias_dt,
                              const void* down, int down_dt, const void* up, int up_dt, const void* h_r,
                              int64_t rank, double scale, const void* dy, int dy_dt, void* dx, void* d_down,
                              void* d_up, int64_t M, int64_t N, int64_t K, void* workspace, size_t workspace_bytes,
                              void* stream) {
    if (w != nullptr && w_t != nullptr) return LYC_ERR_INVALID_ARG;
    const int want = (dx ? BWD_DX : 0) | (d_down ? BWD_DDOWN : 0) | (d_up ? BWD_DUP : 0) | (w_t ? BWD_WT : 0) |
                     (h_r ? BWD_H : 0);
    Bwd B{Problem{true, M, N, K, rank, x_dt, w_dt, bias_dt, down_dt, up_dt, 0, 0, 0}, dy_dt, want, 0};
    const int st = check_bwd(B);
    if (st != LYC_OK) return st;
    return backward(B, x, w, down, up, scale, dy, dx, d_down, d_up, workspace, workspace_bytes, stream, w_t, h_r);
}

int lyc_lora_linear_bwd_workspace_layout(int64_t M, int64_t N, int64_t K, int64_t rank, int x_dt, int w_dt,
                                         int bias_dt, int down_dt, int up_dt, int dy_dt, int want,
                                         size_t* h_offset, size_t* gh_offset, int64_t* ld, size_t* flagged_offset) {
    Bwd B{Problem{true, M, N, K, rank, x_dt, w_dt, bias_dt, down_dt, up_dt, 0, 0, 0}, dy_dt, want, 0};
    const int st = check_bwd(B);
    if (st != LYC_OK) return st;
    const BwdLayout L = bwd_layout(B);
    if (h_offset) *h_offset = L.need_h ? L.h : (size_t)-1;
    if (gh_offset) *gh_offset = L.need_gh ? L.gh : (size_t)-1;
    if (ld) *ld = B.P.r_pad;
    if (flagged_offset) *flagged_offset = L.need_gh && B.P.c_dt != LYC_F32 ? L.flag_g : (size_t)-1;
    return LYC_OK;
}

// ---- DoRA -------------------------------------------------------------------------

int lyc_dora_norms_workspace_size(int64_t N, int64_t K, int64_t rank, int w_dt, int down_dt, int up_dt,
                                  size_t* bytes) {
    Merge G{N, K, rank, w_dt, down_dt, up_dt, 0, 0, 0, 0, 0, 0};
    const int st = check_merge(G);
    if (st != LYC_OK) return st;
    if (bytes) *bytes = align256(G.total) + align256((size_t)((K + 127) / 128) * (size_t)N * 4);
    return LYC_OK;
}

int lyc_dora_norms(const void* w, int w_dt, const void* down, int down_dt, const void* up, int up_dt, int64_t rank,
                   double scale, float* norms, int64_t N, int64_t K, void* workspace, size_t workspace_bytes,
                   void* stream) {
    Merge G{N, K, rank, w_dt, down_dt, up_dt, 0, 0, 0, 0, 0, 0};
    int st = check_merge(G);
    if (st != LYC_OK) return st;
    if (!(scale == scale) || scale > 3.4e38 || scale < -3.4e38) return LYC_ERR_INVALID_ARG;
    if (N == 0) return LYC_OK;
    if (norms == nullptr || (K > 0 && w == nullptr)) return LYC_ERR_INVALID_ARG;
    if (rank > 0 && K > 0 && (down == nullptr || up == nullptr)) return LYC_ERR_INVALID_ARG;
    if (!aligned(norms, 4) || (w && !aligned(w, esize(w_dt)))) return LYC_ERR_UNSUPPORTED;
    if (rank > 0 && (!aligned(down, esize(down_dt)) || !aligned(up, esize(up_dt)))) return LYC_ERR_UNSUPPORTED;
    if (overlaps(norms, (size_t)N * 4, w, (size_t)(N * K) * esize(w_dt))) return LYC_ERR_INVALID_ARG;
    const size_t part = align256(G.total), need = part + align256((size_t)((K + 127) / 128) * (size_t)N * 4);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need || !aligned(workspace, 256))) return LYC_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    char* W = (char*)workspace;
    (void)hipGetLastError();
    if (K == 0) {
        // no columns: every norm is 0 (a transpose of an empty source writes only zeros)
        lyc::TransposeParams tp{norms, LYC_F32, 0, 0, norms, LYC_F32, N, 1};
        return lyc::launch_transpose(tp, s) == hipSuccess ? LYC_OK : LYC_ERR_HIP;
    }
    const bool raw = merge_reads_as_stored(G, down, up);
    lyc::MergeParams mg{};
    mg.w = w;
    mg.w_dt = w_dt;
    mg.dt_c = W + G.dt_c;
    mg.uc = W + G.uc;
    mg.out = nullptr;
    mg.out_dt = G.o_dt;
    mg.N = N;
    mg.K = K;
    mg.r_pad = G.r_pad;
    mg.scale = (float)scale;
    const int E = (w_dt == LYC_F32 || G.o_dt == LYC_F32) ? 4 : 8;
    mg.vec = (K % E == 0) && aligned(w, E * esize(w_dt));
    mg.norm_partial = (float*)(W + part);
    mg.norms = norms;
    if (raw) {
        mg.down_raw = down;
        mg.up_raw = up;
        mg.rank = G.rank;
    }
    if (merge_prepare(G, down, up, raw, W, s) != LYC_OK) return LYC_ERR_HIP;
    if (timed(LYC_KERNEL_GEMM, s, [&] { return lyc::launch_merge(G.c_dt, mg, s); }) != hipSuccess) return LYC_ERR_HIP;
    if (timed(LYC_KERNEL_PREP, s, [&] { return lyc::launch_norm_finish(G.c_dt, mg, s); }) != hipSuccess) return LYC_ERR_HIP;
    return LYC_OK;
}

int lyc_dora_linear_workspace_size(int64_t M, int64_t N, int64_t K, int64_t rank, int x_dt, int w_dt, int bias_dt,
                                   int down_dt, int up_dt, int m_dt, size_t* bytes) {
    Problem P{true, M, N, K, rank, x_dt, w_dt, bias_dt, down_dt, up_dt, 0, 0, 0, m_dt == 0 ? -1 : m_dt};
    const int st = check_problem(P);
    if (st != LYC_OK) return st;
    if (bytes) *bytes = layout(P).total;
    return LYC_OK;
}

int lyc_dora_linear_fwd(const void* x, int x_dt, const void* w, int w_dt, const void* bias, int bias_dt,
                        const void* down, int down_dt, const void* up, int up_dt, const void* magnitude, int m_dt,
                        const float* norms, int64_t rank, double scale, void* y, int y_dt, int64_t M, int64_t N,
                        int64_t K, void* workspace, size_t workspace_bytes, void* stream) {
    Problem P{true, M, N, K, rank, x_dt, w_dt, bias_dt, down_dt, up_dt, 0, 0, 0, m_dt == 0 ? -1 : m_dt};
    const int st = check_problem(P);
    if (st != LYC_OK) return st;
    if (!valid_dt(y_dt)) return LYC_ERR_INVALID_ARG;
    if (!(scale == scale) || scale > 3.4e38 || scale < -3.4e38) return LYC_ERR_INVALID_ARG;
    if (M > 0 && N > 0 && (magnitude == nullptr || norms == nullptr)) return LYC_ERR_INVALID_ARG;
    if ((magnitude && !aligned(magnitude, esize(m_dt))) || (norms && !aligned(norms, 4))) return LYC_ERR_UNSUPPORTED;
    return forward(P, x, w, bias, down, up, scale, y, y_dt, workspace, workspace_bytes, stream, nullptr, magnitude,
                   norms);
}

int lyc_lora_merge_workspace_size(int64_t N, int64_t K, int64_t rank, int w_dt, int down_dt, int up_dt,
                                  size_t* bytes) {
    Merge G{N, K, rank, w_dt, down_dt, up_dt, 0, 0, 0, 0, 0, 0};
    const int st = check_merge(G);
    if (st != LYC_OK) return st;
    if (bytes) *bytes = G.total;
    return LYC_OK;
}

int lyc_lora_merge_fwd(const void* w, int w_dt, const void* down, int down_dt, const void* up, int up_dt,
                       int64_t rank, double scale, void* out, int out_dt, int64_t N, int64_t K, void* workspace,
                       size_t workspace_bytes, void* stream) {
    Merge G{N, K, rank, w_dt, down_dt, up_dt, 0, 0, 0, 0, 0, 0};
    const int st = check_merge(G);
    if (st != LYC_OK) return st;
    if (!valid_dt(out_dt)) return LYC_ERR_INVALID_ARG;
    return merge(G, w, down, up, scale, out, out_dt, workspace, workspace_bytes, stream);
}

int lyc_resolve_dtypes(const int* operand_dtypes, int n, int* compute, int* output) {
    return resolve(operand_dtypes, n, compute, output);
}

int lyc_linear_workspace_size(int64_t M, int64_t N, int64_t K, int x_dt, int w_dt, int bias_dt, size_t* bytes) {
    Problem P{false, M, N, K, 0, x_dt, w_dt, bias_dt, 0, 0, 0, 0, 0};
    const int st = check_problem(P);
    if (st != LYC_OK) return st;
    if (bytes) *bytes = layout(P).total;
    return LYC_OK;
}

int lyc_linear_fwd(const void* x, int x_dt, const void* w, int w_dt, const void* bias, int bias_dt, void* y,
                   int y_dt, int64_t M, int64_t N, int64_t K, void* workspace, size_t workspace_bytes,
                   void* stream) {
    Problem P{false, M, N, K, 0, x_dt, w_dt, bias_dt, 0, 0, 0, 0, 0};
    const int st = check_problem(P);
    if (st != LYC_OK) return st;
    if (!valid_dt(y_dt)) return LYC_ERR_INVALID_ARG;
    return forward(P, x, w, bias, nullptr, nullptr, 1.0, y, y_dt, workspace, workspace_bytes, stream);
}

int lyc_linear_prepare(const void* w, int w_dt, int x_dt, int bias_dt, int64_t M, int64_t N, int64_t K,
                       void* workspace, size_t workspace_bytes, void* stream) {
    Problem P{false, M, N, K, 0, x_dt, w_dt, bias_dt, 0, 0, 0, 0, 0};
    const int st = check_problem(P);
    if (st != LYC_OK) return st;
    if (P.M == 0 || P.N == 0 || P.K == 0) return LYC_OK;
    if (w == nullptr) return LYC_ERR_INVALID_ARG;
    if (!aligned(w, 16)) return LYC_ERR_UNSUPPORTED;
    const Layout L = layout(P);
    if (L.total > 0 && (workspace == nullptr || workspace_bytes < L.total || !aligned(workspace, 256)))
        return LYC_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    char* W = (char*)workspace;
    (void)hipGetLastError();
    const void* wa = w;
    if (L.cast_w) {
        wa = W + L.wc;
        if (timed(LYC_KERNEL_CAST, s, [&] { return lyc::launch_cast((const float*)w, W + L.wc, P.N * P.K, P.c_dt, s); }) !=
            hipSuccess)
            return LYC_ERR_HIP;
    }
    if (L.w_split_pass && timed(LYC_KERNEL_PREP, s, [&] {
            return lyc::launch_rownorm(wa, P.c_dt, P.N, P.K, W + L.wh, W + L.wl, (double2*)(W + L.wnorm), nullptr, s);
        }) != hipSuccess)
        return LYC_ERR_HIP;
    return LYC_OK;
}

int lyc_linear_fwd_prepared(const void* x, int x_dt, const void* w, int w_dt, const void* bias, int bias_dt, void* y,
                            int y_dt, int64_t M, int64_t N, int64_t K, void* workspace, size_t workspace_bytes,
                            void* stream) {
    Problem P{false, M, N, K, 0, x_dt, w_dt, bias_dt, 0, 0, 0, 0, 0};
    const int st = check_problem(P);
    if (st != LYC_OK) return st;
    if (!valid_dt(y_dt)) return LYC_ERR_INVALID_ARG;
    P.w_prepared = true;
    return forward(P, x, w, bias, nullptr, nullptr, 1.0, y, y_dt, workspace, workspace_bytes, stream);
}

int lyc_lora_linear_workspace_size(int64_t M, int64_t N, int64_t K, int64_t rank, int x_dt, int w_dt, int bias_dt,
                                   int down_dt, int up_dt, size_t* bytes) {
    Problem P{true, M, N, K, rank, x_dt, w_dt, bias_dt, down_dt, up_dt, 0, 0, 0};
    const int st = check_problem(P);
    if (st != LYC_OK) return st;
    if (bytes) *bytes = layout(P).total;
    return LYC_OK;
}

int lyc_lora_linear_fwd(const void* x, int x_dt, const void* w, int w_dt, const void* bias, int bias_dt,
                        const void* down, int down_dt, const void* up, int up_dt, int64_t rank, double scale,
                        void* y, int y_dt, int64_t M, int64_t N, int64_t K, void* workspace,
                        size_t workspace_bytes, void* stream) {
    Problem P{true, M, N, K, rank, x_dt, w_dt, bias_dt, down_dt, up_dt, 0, 0, 0};
    const int st = check_problem(P);
    if (st != LYC_OK) return st;
    if (!valid_dt(y_dt)) return LYC_ERR_INVALID_ARG;
    if (!(scale == scale) || scale > 3.4e38 || scale < -3.4e38) return LYC_ERR_INVALID_ARG;
    return forward(P, x, w, bias, down, up, scale, y, y_dt, workspace, workspace_bytes, stream);
}

int lyc_lora_linear_wc_workspace_size(int64_t M, int64_t N, int64_t K, int64_t rank, int x_dt, int w_dt,
                                      int bias_dt, int down_dt, int up_dt, size_t* bytes) {
    Problem P{true, M, N, K, rank, x_dt, w_dt, bias_dt, down_dt, up_dt, 0, 0, 0};
    P.w_kept = true;
    const int st = check_problem(P);
    if (st != LYC_OK) return st;
    if (bytes) *bytes = layout(P).total;
    return LYC_OK;
}

int lyc_lora_linear_fwd_wc(const void* x, int x_dt, const void* w_c, int w_dt, const void* bias, int bias_dt,
                           const void* down, int down_dt, const void* up, int up_dt, int64_t rank, double scale,
                           void* y, int y_dt, int64_t M, int64_t N, int64_t K, void* workspace,
                           size_t workspace_bytes, void* stream) {
    Problem P{true, M, N, K, rank, x_dt, w_dt, bias_dt, down_dt, up_dt, 0, 0, 0};
    P.w_kept = true;
    const int st = check_problem(P);
    if (st != LYC_OK) return st;
    if (!valid_dt(y_dt)) return LYC_ERR_INVALID_ARG;
    if (!(scale == scale) || scale > 3.4e38 || scale < -3.4e38) return LYC_ERR_INVALID_ARG;
    return forward(P, x, w_c, bias, down, up, scale, y, y_dt, workspace, workspace_bytes, stream);
}

int lyc_lora_workspace_layout(int64_t M, int64_t N, int64_t K, int64_t rank, int x_dt, int w_dt, int bias_dt,
                              int down_dt, int up_dt, size_t* h_offset, int64_t* h_ld, size_t* flagged_offset,
                              int64_t* flagged_slots) {
    Problem P{true, M, N, K, rank, x_dt, w_dt, bias_dt, down_dt, up_dt, 0, 0, 0};
    const int st = check_problem(P);
    if (st != LYC_OK) return st;
    const Layout L = layout(P);
    if (h_offset) *h_offset = L.h;
    if (h_ld) *h_ld = P.r_pad;
    if (flagged_offset) *flagged_offset = L.flagged;
    if (flagged_slots) *flagged_slots = L.flag_slots;
    return LYC_OK;
}

int lyc_linear_workspace_layout(int64_t M, int64_t N, int64_t K, int x_dt, int w_dt, int bias_dt,
                                size_t* flagged_offset, int64_t* flagged_slots) {
    Problem P{false, M, N, K, 0, x_dt, w_dt, bias_dt, 0, 0, 0, 0, 0};
    const int st = check_problem(P);
    if (st != LYC_OK) return st;
    const Layout L = layout(P);
    if (flagged_offset) *flagged_offset = L.flagged;
    if (flagged_slots) *flagged_slots = L.flag_slots;
    return LYC_OK;
}

int lyc_profile_begin(int capacity) {
    if (capacity < 1) return LYC_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    for (auto& p : g_prof) {
        (void)hipEventDestroy(p.a);
        (void)hipEventDestroy(p.b);
    }
    g_prof.clear();
    g_prof_used = 0;
    g_prof_on = false;
    for (int i = 0; i < capacity; ++i) {
        ProfSlot p{};
        if (hipEventCreate(&p.a) != hipSuccess) return LYC_ERR_HIP;
        if (hipEventCreate(&p.b) != hipSuccess) {
            (void)hipEventDestroy(p.a);
            return LYC_ERR_HIP;
        }
        g_prof.push_back(p);
    }
    g_prof_on = true;
    return LYC_OK;
}

int lyc_profile_end(double* total_ms, int* launches) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    double t[LYC_KERNEL_KINDS] = {};
    int n[LYC_KERNEL_KINDS] = {};
    int st = LYC_OK;
    for (size_t i = 0; i < g_prof_used; ++i) {
        float ms = 0.f;
        if (hipEventSynchronize(g_prof[i].b) != hipSuccess ||
            hipEventElapsedTime(&ms, g_prof[i].a, g_prof[i].b) != hipSuccess) {
            st = LYC_ERR_HIP;
            continue;
        }
        t[g_prof[i].kind] += ms;
        n[g_prof[i].kind] += 1;
    }
    for (auto& p : g_prof) {
        (void)hipEventDestroy(p.a);
        (void)hipEventDestroy(p.b);
    }
    g_prof.clear();
    g_prof_used = 0;
    g_prof_on = false;
    for (int k = 0; k < LYC_KERNEL_KINDS; ++k) {
        if (total_ms) total_ms[k] = t[k];
        if (launches) launches[k] = n[k];
    }
    return st;
}

int lyc_gemm_tile(int64_t M, int64_t N, int compute_dt, int* tile_n, int* tile_m) {
    if (M < 0 || N < 0 || !valid_dt(compute_dt)) return LYC_ERR_INVALID_ARG;
    int tn = 0, tm = 0;
    lyc::gemm_tile_shape(M, N, compute_dt, &tn, &tm);
    if (tile_n) *tile_n = tn;
    if (tile_m) *tile_m = tm;
    return LYC_OK;
}

const char* lyc_status_str(int status) {
    switch (status) {
    case LYC_OK: return "ok";
    case LYC_ERR_MIXED_HALF: return "fp16 and bf16 operands in one call (no common 16-bit type; refused)";
    case LYC_ERR_INVALID_ARG: return "invalid argument";
    case LYC_ERR_DTYPE_MISMATCH: return "output dtype differs from the resolved output dtype";
    case LYC_ERR_UNSUPPORTED: return "unsupported shape, alignment or rank";
    case LYC_ERR_HIP: return "HIP runtime error while launching";
    case LYC_ERR_WORKSPACE: return "workspace missing, too small or not 256-byte aligned";
    case LYC_ERR_IO: return "tuning table file could not be read, parsed or written";
    case LYC_ERR_SCRATCH: return "the problem needs more scratch than the allocation-free forward holds";
    default: return "unknown status";
    }
}

}  // extern "C"
