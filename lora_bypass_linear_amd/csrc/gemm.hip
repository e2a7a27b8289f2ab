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
//   2. main               acc += x_c . W_c^T     K loop, multi-stage LDS pipeline
//   3. epilogue           y = round_out(acc + b), one rounding
//
// Accumulation is fp32 throughout (LyCORIS "Precision" page, "Dtype policy");
// the bypass lands in the same accumulators as x.W^T, so Delta W = up.down is
// never formed ("VRAM" section).
#include "kernels.h"
#include "lyc_device.h"

namespace lyc {

// TN x TM output tile, WN x WM per wave (multiples of 16), NS pipeline stages
// of one K step each; a K step is 64 bytes of every row (32 16-bit values).
template <int TN_, int TM_, int WN_, int WM_, int NS_>
struct Tile {
    static constexpr int TN = TN_, TM = TM_, WN = WN_, WM = WM_, NS = NS_;
    static constexpr int WAVES_N = TN / WN, WAVES_M = TM / WM;
    static constexpr int NW = WAVES_N * WAVES_M, NT = NW * 64;
    static constexpr int FN = WN / 16, FM = WM / 16;
    static constexpr int NBLK = (TN + TM) / 16;                 // 1 KiB LDS blocks (16 rows) per step
    static constexpr int QMAX = (NBLK + NW - 1) / NW;           // loads per wave per step, at most
    static constexpr int QMIN = NBLK / NW;                      // ... at least
    static constexpr int STAGE = (TN + TM) * 64;                // LDS bytes per stage
    static_assert(TN % WN == 0 && TM % WM == 0 && WN % 16 == 0 && WM % 16 == 0, "tile shape");
    static_assert(TN % 16 == 0 && TM % 16 == 0 && QMIN >= 1, "loader split");
    static_assert(NS * STAGE <= 160 * 1024, "LDS");
};

using TileL = Tile<256, 256, 128, 64, 4>;  // 8 waves, 128 KiB
using TileG = Tile<192, 256, 96, 64, 5>;   // 8 waves, 140 KiB
using TileM = Tile<128, 128, 64, 64, 4>;   // 4 waves, 64 KiB
using TileS = Tile<64, 64, 32, 32, 4>;     // 4 waves, 32 KiB

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

// LDS rows are 64 bytes (4 chunks of 16); chunk kc of row r sits at slot
// kc ^ ((r >> 1) & 3), so the 16-byte fragment reads of 8 consecutive rows
// (two rows per 128 bytes) hit 8 different bank groups.
__device__ __forceinline__ int lds64(int row, int kc) { return row * 64 + ((kc ^ ((row >> 1) & 3)) << 4); }

// Global -> LDS without registers: one buffer_load_dwordx4 ... lds per wave
// fills 1 KiB of LDS = 16 rows x 64 bytes of a K step.  The LDS side of such a
// load is fixed (lane l writes bytes 16l .. 16l+15 of the KiB), so each lane
// fetches the global chunk that belongs in that slot of the swizzled layout:
// row 16 blk + (l >> 2), logical chunk (l & 3) ^ ((l >> 3) & 3).  The blocks of
// the A (W-side) and B (x-side) tiles are numbered together and dealt to the
// waves round-robin.
template <class TL>
struct Loader {
    uint32_t vo[TL::QMAX];
    __device__ __forceinline__ void init(uint32_t a_bytes, uint32_t b_bytes, int wave, int lane) {
        const uint32_t kc16 = (uint32_t)((lane & 3) ^ ((lane >> 3) & 3)) << 4;
#pragma unroll
        for (int q = 0; q < TL::QMAX; ++q) {
            const int blk = wave + q * TL::NW;
            const bool is_a = blk < TL::TN / 16;
            const int row = (is_a ? blk : blk - TL::TN / 16) * 16 + (lane >> 2);
            vo[q] = (uint32_t)row * (is_a ? a_bytes : b_bytes) + kc16;
        }
    }
    // loads of one K step (kb0 = its first byte within a row) into an LDS stage;
    // rows past a tile's valid rows read zeros through the buffer range check, and
    // in the last, ragged step the chunks past K are sent out of range too
    __device__ __forceinline__ void issue(char* stage, __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb,
                                          uint32_t row_bytes, uint32_t kb0, int wave, int lane) const {
        const bool full = kb0 + 64 <= row_bytes;
        const uint32_t kc16 = (uint32_t)((lane & 3) ^ ((lane >> 3) & 3)) << 4;
#pragma unroll
        for (int q = 0; q < TL::QMAX; ++q) {
            const int blk = wave + q * TL::NW;
            if (q >= TL::QMIN && blk >= TL::NBLK) break;
            uint32_t v = vo[q];
            if (!full) v = (kb0 + kc16 < row_bytes) ? v : OOB;
            // (an if, not ?:, on the resource: the host pass silently drops the
            // kernel stub for a conditional over __amdgpu_buffer_rsrc_t)
            auto* dst = (__attribute__((address_space(3))) void*)(stage + blk * 1024);
            if (blk < TL::TN / 16) __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, dst, 16, v, (int)kb0, 0, 0);
            else __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, dst, 16, v, (int)kb0, 0, 0);
        }
    }
};

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima)
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Workgroup barrier that orders LDS only.  A __syncthreads() also waits for
// every outstanding global load (vmcnt(0)), which defeats loads issued several
// steps ahead; here the wave's own LDS reads are drained (lgkmcnt(0)), so a
// stage read before the barrier may be refilled after it, and completion of
// its own LDS-bound loads is established by an explicit wait_vm before it.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0), vmcnt and expcnt unconstrained
    asm volatile("s_barrier" ::: "memory");
}

// This wave's operand fragments of one K step (64 bytes per row) from an LDS
// stage: FN 16-row blocks of the A tile, FM of the B tile.
template <class TL>
__device__ __forceinline__ void read_frags(const char* st, i32x4 (&fa)[TL::FN], i32x4 (&fb)[TL::FM], int lane,
                                           int wn, int wm) {
    const int kc = lane >> 4;
    const char* sb = st + TL::TN * 64;
#pragma unroll
    for (int i = 0; i < TL::FN; ++i) fa[i] = *(const i32x4*)(st + lds64(wn * TL::WN + i * 16 + (lane & 15), kc));
#pragma unroll
    for (int j = 0; j < TL::FM; ++j) fb[j] = *(const i32x4*)(sb + lds64(wm * TL::WM + j * 16 + (lane & 15), kc));
}

template <class CT, class TL>
__device__ __forceinline__ void mma(const i32x4 (&fa)[TL::FN], const i32x4 (&fb)[TL::FM],
                                    f32x4 (&acc)[TL::FN][TL::FM]) {
#pragma unroll
    for (int i = 0; i < TL::FN; ++i)
#pragma unroll
        for (int j = 0; j < TL::FM; ++j) acc[i][j] = CT::step(fa[i], fb[j], acc[i][j]);
}

// The K steps of one tile: first the fold steps over the padded rank (A = up_c,
// B = h_r), then the main steps over K (A = W_c, B = x_c).
template <class TL>
struct Steps {
    Loader<TL> lf, lm;
    __amdgpu_buffer_rsrc_t fa, fb, ma, mb;
    uint32_t fbytes, kbytes;
    int RF, KT;
    __device__ __forceinline__ void issue(char* smem, int s, int wave, int lane) const {
        char* st = smem + (s % TL::NS) * TL::STAGE;
        if (s < RF) lf.issue(st, fa, fb, fbytes, (uint32_t)s * 64, wave, lane);
        else lm.issue(st, ma, mb, kbytes, (uint32_t)(s - RF) * 64, wave, lane);
    }
};

// One pipeline step kt: wait until step kt+1 has landed in LDS (steps up to
// kt+NS-1 are in flight), barrier, refill the stage of step kt (its fragments
// are already in registers) with step kt+NS, read step kt+1's fragments into
// (nfa, nfb) while the MFMAs of step kt run on (cfa, cfb).
template <class CT, class TL>
__device__ __forceinline__ void pipe_step(const Steps<TL>& S, char* smem, int kt, const i32x4 (&cfa)[TL::FN],
                                          const i32x4 (&cfb)[TL::FM], i32x4 (&nfa)[TL::FN], i32x4 (&nfb)[TL::FM],
                                          f32x4 (&acc)[TL::FN][TL::FM], int wave, int lane, int wn, int wm) {
    if (kt + TL::NS - 1 < S.KT) wait_vm<(TL::NS - 2) * TL::QMIN>();
    else wait_vm<0>();
    lds_barrier();
    if (kt + TL::NS < S.KT) S.issue(smem, kt + TL::NS, wave, lane);
    if (kt + 1 < S.KT) read_frags<TL>(smem + ((kt + 1) % TL::NS) * TL::STAGE, nfa, nfb, lane, wn, wm);
    __builtin_amdgcn_s_setprio(1);
    mma<CT, TL>(cfa, cfb, acc);
    __builtin_amdgcn_s_setprio(0);
}

// Steps [kt, end) of the pipeline, two per iteration so that the register sets
// alternate statically; on return the fragments of step `end` are in (fa0, fb0).
template <class CT, class TL>
__device__ __forceinline__ void pipe_run(const Steps<TL>& S, char* smem, int kt, int end, i32x4 (&fa0)[TL::FN],
                                         i32x4 (&fb0)[TL::FM], i32x4 (&fa1)[TL::FN], i32x4 (&fb1)[TL::FM],
                                         f32x4 (&acc)[TL::FN][TL::FM], int wave, int lane, int wn, int wm) {
    for (; kt + 1 < end; kt += 2) {
        pipe_step<CT, TL>(S, smem, kt, fa0, fb0, fa1, fb1, acc, wave, lane, wn, wm);
        pipe_step<CT, TL>(S, smem, kt + 1, fa1, fb1, fa0, fb0, acc, wave, lane, wn, wm);
    }
    if (kt < end) {
        pipe_step<CT, TL>(S, smem, kt, fa0, fb0, fa1, fb1, acc, wave, lane, wn, wm);
#pragma unroll
        for (int i = 0; i < TL::FN; ++i) fa0[i] = fa1[i];
#pragma unroll
        for (int j = 0; j < TL::FM; ++j) fb0[j] = fb1[j];
    }
}

template <class CT, class TL>
__global__ __launch_bounds__(TL::NT, 1) void gemm_kernel(GemmParams p, int tiles_n, int tiles_m, int group_m) {
    __shared__ __attribute__((aligned(16))) char smem[TL::NS * TL::STAGE];
    constexpr int FN = TL::FN, FM = TL::FM;
    const int tid = threadIdx.x, lane = tid & 63;
    // wave index in a scalar register: everything derived from it stays uniform
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    (void)tid;
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

    // 1-2. fold and main contraction in one pipeline of K steps: NS LDS stages
    //      filled straight from global memory, NS steps ahead of their use;
    //      fragments are read one step ahead into a second register set.
    Steps<TL> S;
    S.fbytes = (uint32_t)(p.rf * CT::es);
    S.kbytes = (uint32_t)(p.K * CT::es);
    S.RF = (int)(S.fbytes / 64);
    S.KT = S.RF + (int)((S.kbytes + 63) / 64);
    S.fa = make_rsrc((const char*)p.af + n0 * S.fbytes, (uint32_t)rows_a * S.fbytes);
    S.fb = make_rsrc((const char*)p.bf + m0 * S.fbytes, (uint32_t)rows_b * S.fbytes);
    S.ma = make_rsrc((const char*)p.a + n0 * S.kbytes, (uint32_t)rows_a * S.kbytes);
    S.mb = make_rsrc((const char*)p.b + m0 * S.kbytes, (uint32_t)rows_b * S.kbytes);
    S.lf.init(S.fbytes, S.fbytes, wave, lane);
    S.lm.init(S.kbytes, S.kbytes, wave, lane);
    const int KT = S.KT;
    if (KT > 0) {
        i32x4 fa0[FN], fb0[FM], fa1[FN], fb1[FM];
#pragma unroll
        for (int s0 = 0; s0 < TL::NS; ++s0)
            if (s0 < KT) S.issue(smem, s0, wave, lane);
        if (TL::NS - 1 < KT) wait_vm<(TL::NS - 1) * TL::QMIN>();
        else wait_vm<0>();
        lds_barrier();
        read_frags<TL>(smem, fa0, fb0, lane, wn, wm);
        // fold steps, then acc = scale * (h_r . up_c^T) once, then the main steps:
        // the accumulators see no vector ALU work inside either loop
        pipe_run<CT, TL>(S, smem, 0, S.RF, fa0, fb0, fa1, fb1, acc, wave, lane, wn, wm);
        if (S.RF > 0) {
#pragma unroll
            for (int i = 0; i < FN; ++i)
#pragma unroll
                for (int j = 0; j < FM; ++j) acc[i][j] *= p.scale;
        }
        pipe_run<CT, TL>(S, smem, S.RF, KT, fa0, fb0, fa1, fb1, acc, wave, lane, wn, wm);
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
    hipLaunchKernelGGL((gemm_kernel<CT, TL>), dim3(nblk), dim3(TL::NT), 0, s, p, tiles_n, tiles_m, 4);
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
