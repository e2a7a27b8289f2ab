// gemm.hip -- the main contraction of the LoRA-bypass linear on gfx950 MFMA.
//
// One workgroup owns one output tile y[m0:m0+TM, n0:n0+TN].  The A side of
// every MFMA is a weight-shaped operand indexed by n (W_c, up_c), the B side an
// activation-shaped operand indexed by m (x_c, h_r); both are K-contiguous
// ("TN"), so 16-byte global loads and 16-byte LDS fragment reads feed the
// MFMAs without any transpose.
//
//   1. fold   (LoRA only)  acc  = h_r . up_c^T   over the padded rank, then
//                          acc *= scale          (one fp32 multiply)
//   2. main               acc += x_c . W_c^T     K loop, LDS double buffer
//   3. epilogue           y = round_out(acc + b), one rounding
//
// Accumulation is fp32 throughout (LyCORIS "Precision" page, "Dtype policy");
// the bypass lands in the same accumulators as x.W^T, so Delta W = up.down is
// never formed ("VRAM" section).
#include "kernels.h"
#include "lyc_device.h"

namespace lyc {

// TN x TM output tile, WN x WM per wave (multiples of 16), K step of 128 bytes.
template <int TN_, int TM_, int WN_, int WM_>
struct Tile {
    static constexpr int TN = TN_, TM = TM_, WN = WN_, WM = WM_;
    static constexpr int WAVES_N = TN / WN, WAVES_M = TM / WM;
    static constexpr int NW = WAVES_N * WAVES_M, NT = NW * 64;
    static constexpr int FN = WN / 16, FM = WM / 16;
    static constexpr int CA = TN * 8 / NT, CB = TM * 8 / NT;  // 16-byte chunks per thread per K step
    static constexpr int STAGE = (TN + TM) * 128;              // LDS bytes per pipeline stage
    static_assert(TN % WN == 0 && TM % WM == 0 && WN % 16 == 0 && WM % 16 == 0, "tile shape");
    static_assert((TN * 8) % NT == 0 && (TM * 8) % NT == 0, "loader split");
};

using TileL = Tile<256, 256, 128, 64>;  // 8 waves
using TileG = Tile<192, 256, 96, 64>;   // 8 waves
using TileM = Tile<128, 128, 64, 64>;   // 4 waves
using TileS = Tile<64, 64, 32, 32>;     // 4 waves

// Workgroup id -> output tile.  Workgroups are dispatched round-robin over the
// 8 XCDs (id % 8), each with its own L2: give every XCD a contiguous range of
// logical tiles, and walk that range in groups of `group_m` m-tiles so the
// tiles resident on one XCD share W and x rows in its L2.
__device__ __forceinline__ void tile_coords(int bid, int nblk, int tiles_n, int tiles_m, int group_m, int& tn,
                                            int& tm) {
    const int per = nblk >> 3, rem = nblk & 7;
    const int xcd = bid & 7, loc = bid >> 3;
    const int l = xcd * per + (xcd < rem ? xcd : rem) + loc;
    const int in_group = group_m * tiles_n;
    const int g = l / in_group;
    const int first_m = g * group_m;
    const int gsz = (tiles_m - first_m) < group_m ? (tiles_m - first_m) : group_m;
    const int r = l - g * in_group;
    tm = first_m + r % gsz;
    tn = r / gsz;
}

template <int CH, int NT>
__device__ __forceinline__ void load_chunks(i32x4 (&reg)[CH], __amdgpu_buffer_rsrc_t rs, uint32_t row_bytes,
                                            uint32_t kb0, int tid) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
        const int c = tid + i * NT;
        const uint32_t kb = kb0 + ((c & 7) << 4);
        const uint32_t off = kb < row_bytes ? (uint32_t)(c >> 3) * row_bytes + kb : OOB;
        reg[i] = buf_load16(rs, off);
    }
}

template <int CH, int NT>
__device__ __forceinline__ void store_chunks(char* lds, const i32x4 (&reg)[CH], int tid) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
        const int c = tid + i * NT;
        *(i32x4*)(lds + lds_off(c >> 3, c & 7)) = reg[i];
    }
}

// MFMAs over one 128-byte K step held in LDS (two 64-byte halves).
template <class CT, class TL>
__device__ __forceinline__ void mma_stage(const char* sa, const char* sb, f32x4 (&acc)[TL::FN][TL::FM], int lane,
                                          int wn, int wm) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        i32x4 fa[TL::FN], fb[TL::FM];
        const int kc = s * 4 + (lane >> 4);
#pragma unroll
        for (int i = 0; i < TL::FN; ++i) fa[i] = *(const i32x4*)(sa + lds_off(wn * TL::WN + i * 16 + (lane & 15), kc));
#pragma unroll
        for (int j = 0; j < TL::FM; ++j) fb[j] = *(const i32x4*)(sb + lds_off(wm * TL::WM + j * 16 + (lane & 15), kc));
#pragma unroll
        for (int i = 0; i < TL::FN; ++i)
#pragma unroll
            for (int j = 0; j < TL::FM; ++j) acc[i][j] = CT::step(fa[i], fb[j], acc[i][j]);
    }
}

template <class CT, class TL>
__global__ __launch_bounds__(TL::NT, 1) void gemm_kernel(GemmParams p, int tiles_n, int tiles_m, int group_m) {
    __shared__ __attribute__((aligned(16))) char smem[2 * TL::STAGE];
    constexpr int NT = TL::NT, FN = TL::FN, FM = TL::FM;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wn = wave % TL::WAVES_N, wm = wave / TL::WAVES_N;
    int tn, tm;
    tile_coords(blockIdx.x, gridDim.x, tiles_n, tiles_m, group_m, tn, tm);
    const int64_t n0 = (int64_t)tn * TL::TN, m0 = (int64_t)tm * TL::TM;
    const int rows_a = (int)((p.N - n0) < TL::TN ? (p.N - n0) : TL::TN);
    const int rows_b = (int)((p.M - m0) < TL::TM ? (p.M - m0) : TL::TM);

    f32x4 acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    char* const st0 = smem;
    char* const st1 = smem + TL::STAGE;
    i32x4 ra[TL::CA], rb[TL::CB];

    // 1. fold: acc = scale * (h_r . up_c^T)
    if (p.rf > 0) {
        const uint32_t fb = (uint32_t)(p.rf * CT::es);
        const auto rsa = make_rsrc((const char*)p.af + n0 * fb, (uint32_t)rows_a * fb);
        const auto rsb = make_rsrc((const char*)p.bf + m0 * fb, (uint32_t)rows_b * fb);
        for (uint32_t kb = 0; kb < fb; kb += 128) {
            load_chunks<TL::CA, NT>(ra, rsa, fb, kb, tid);
            load_chunks<TL::CB, NT>(rb, rsb, fb, kb, tid);
            store_chunks<TL::CA, NT>(st0, ra, tid);
            store_chunks<TL::CB, NT>(st0 + TL::TN * 128, rb, tid);
            __syncthreads();
            mma_stage<CT, TL>(st0, st0 + TL::TN * 128, acc, lane, wn, wm);
            __syncthreads();
        }
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int j = 0; j < FM; ++j) acc[i][j] *= p.scale;
    }

    // 2. main K loop: two LDS stages, and global loads issued two K steps ahead
    //    into alternating register sets, so a load has a full compute phase of
    //    the previous step plus its own to arrive.
    const uint32_t kbytes = (uint32_t)(p.K * CT::es);
    if (kbytes > 0) {
        const auto rsa = make_rsrc((const char*)p.a + n0 * kbytes, (uint32_t)rows_a * kbytes);
        const auto rsb = make_rsrc((const char*)p.b + m0 * kbytes, (uint32_t)rows_b * kbytes);
        const int KT = (int)((kbytes + 127) / 128);
        i32x4 ra2[TL::CA], rb2[TL::CB];
        load_chunks<TL::CA, NT>(ra, rsa, kbytes, 0, tid);
        load_chunks<TL::CB, NT>(rb, rsb, kbytes, 0, tid);
        if (KT > 1) {
            load_chunks<TL::CA, NT>(ra2, rsa, kbytes, 128, tid);
            load_chunks<TL::CB, NT>(rb2, rsb, kbytes, 128, tid);
        }
        store_chunks<TL::CA, NT>(st0, ra, tid);
        store_chunks<TL::CB, NT>(st0 + TL::TN * 128, rb, tid);
        __syncthreads();
        // invariant at the top of step kt: LDS stage kt&1 holds step kt; the
        // register set (kt+1)&1 holds (or is receiving) step kt+1
        for (int kt = 0; kt < KT; kt += 2) {
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int k = kt + half;
                if (k >= KT) break;
                char* cur = half ? st1 : st0;
                char* nxt = half ? st0 : st1;
                i32x4(&rn_a)[TL::CA] = half ? ra2 : ra;      // receives step k+2
                i32x4(&rn_b)[TL::CB] = half ? rb2 : rb;
                i32x4(&rs_a)[TL::CA] = half ? ra : ra2;      // holds step k+1
                i32x4(&rs_b)[TL::CB] = half ? rb : rb2;
                if (k + 2 < KT) {
                    load_chunks<TL::CA, NT>(rn_a, rsa, kbytes, (uint32_t)(k + 2) * 128, tid);
                    load_chunks<TL::CB, NT>(rn_b, rsb, kbytes, (uint32_t)(k + 2) * 128, tid);
                }
                __builtin_amdgcn_s_setprio(1);
                mma_stage<CT, TL>(cur, cur + TL::TN * 128, acc, lane, wn, wm);
                __builtin_amdgcn_s_setprio(0);
                if (k + 1 < KT) {
                    store_chunks<TL::CA, NT>(nxt, rs_a, tid);
                    store_chunks<TL::CB, NT>(nxt + TL::TN * 128, rs_b, tid);
                }
                __syncthreads();
            }
        }
    }

    // 3. epilogue: lane holds, per 16x16 block, 4 consecutive n for one m
#pragma unroll
    for (int i = 0; i < FN; ++i) {
        const int64_t nb = n0 + wn * TL::WN + i * 16 + 4 * (lane >> 4);
        float bias[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            bias[e] = (p.bias != nullptr && nb + e < p.N) ? load_as_f32(p.bias, p.bias_dt, nb + e) : 0.f;
#pragma unroll
        for (int j = 0; j < FM; ++j) {
            const int64_t m = m0 + wm * TL::WM + j * 16 + (lane & 15);
            if (m >= p.M) continue;
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float a = acc[i][j][e];
                v[e] = a + bias[e];
            }
            const int64_t base = m * p.N + nb;
            if (p.y_dt == DT_F32) {
                float* y = (float*)p.y;
                if (p.vec_store && nb + 3 < p.N) {
                    *(f32x4*)(y + base) = f32x4{v[0], v[1], v[2], v[3]};
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (nb + e < p.N) y[base + e] = v[e];
                }
            } else {
                uint16_t o[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = p.y_dt == DT_F16 ? f32_to_f16(v[e]) : f32_to_bf16(v[e]);
                uint16_t* y = (uint16_t*)p.y;
                if (p.vec_store && nb + 3 < p.N) {
                    *(i32x2*)(y + base) = i32x2{(int)(o[0] | ((uint32_t)o[1] << 16)),
                                                (int)(o[2] | ((uint32_t)o[3] << 16))};
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (nb + e < p.N) y[base + e] = o[e];
                }
            }
        }
    }
}

template <class CT, class TL>
static hipError_t run(const GemmParams& p, hipStream_t s) {
    const int tiles_n = (int)((p.N + TL::TN - 1) / TL::TN);
    const int tiles_m = (int)((p.M + TL::TM - 1) / TL::TM);
    const int nblk = tiles_n * tiles_m;
    hipLaunchKernelGGL((gemm_kernel<CT, TL>), dim3(nblk), dim3(TL::NT), 0, s, p, tiles_n, tiles_m, 8);
    return hipGetLastError();
}

// Tile choice: fewest "rounds" of workgroups over 256 CUs, weighted by tile
// area and a per-shape efficiency penalty (smaller tiles re-read more).
enum { T_L, T_G, T_M, T_S };
static int pick_tile(int64_t M, int64_t N, bool f32) {
    struct C { int id, tn, tm; double pen; };
    const C cands16[] = {{T_L, 256, 256, 1.0}, {T_G, 192, 256, 1.0}, {T_M, 128, 128, 1.3}, {T_S, 64, 64, 2.0}};
    const C cands32[] = {{T_M, 128, 128, 1.0}, {T_S, 64, 64, 1.5}};
    const C* c = f32 ? cands32 : cands16;
    const int nc = f32 ? 2 : 4;
    int best = c[0].id;
    double best_cost = 1e300;
    for (int i = 0; i < nc; ++i) {
        const double tiles = (double)((N + c[i].tn - 1) / c[i].tn) * (double)((M + c[i].tm - 1) / c[i].tm);
        const double rounds = (double)(int64_t)((tiles + 255) / 256);
        const double cost = rounds * c[i].tn * c[i].tm * c[i].pen;
        if (cost < best_cost) { best_cost = cost; best = c[i].id; }
    }
    return best;
}

void gemm_tile_shape(int64_t M, int64_t N, int c_dt, int* tn, int* tm) {
    static const int shape[4][2] = {{256, 256}, {192, 256}, {128, 128}, {64, 64}};
    const int t = pick_tile(M, N, c_dt == DT_F32);
    *tn = shape[t][0];
    *tm = shape[t][1];
}

hipError_t launch_gemm(int c_dt, const GemmParams& p, hipStream_t s) {
    const int t = pick_tile(p.M, p.N, c_dt == DT_F32);
    if (c_dt == DT_F16) {
        switch (t) {
        case T_L: return run<CF16, TileL>(p, s);
        case T_G: return run<CF16, TileG>(p, s);
        case T_M: return run<CF16, TileM>(p, s);
        default: return run<CF16, TileS>(p, s);
        }
    }
    if (c_dt == DT_BF16) {
        switch (t) {
        case T_L: return run<CBF16, TileL>(p, s);
        case T_G: return run<CBF16, TileG>(p, s);
        case T_M: return run<CBF16, TileM>(p, s);
        default: return run<CBF16, TileS>(p, s);
        }
    }
    if (t == T_M) return run<CF32, TileM>(p, s);
    return run<CF32, TileS>(p, s);
}

}  // namespace lyc
