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
#include <algorithm>
#include <cmath>
#include <map>
#include <mutex>

#include "kernels.h"
#include "lyc_device.h"

namespace lyc {

// TN x TM output tile, WN x WM per wave (multiples of 16), NS pipeline stages
// of one K step each.  A K step is BKB bytes of every row (64: 32 16-bit
// values; 128: 64), made of SUB = BKB/64 MFMA substeps of 64 bytes.
template <int TN_, int TM_, int WN_, int WM_, int NS_, int BKB_>
struct Tile {
    static constexpr int TN = TN_, TM = TM_, WN = WN_, WM = WM_, NS = NS_, BKB = BKB_;
    static constexpr int WAVES_N = TN / WN, WAVES_M = TM / WM;
    static constexpr int NW = WAVES_N * WAVES_M, NT = NW * 64;
    static constexpr int FN = WN / 16, FM = WM / 16;
    static constexpr int SUB = BKB / 64;                        // MFMA substeps per K step
    static constexpr int CH = BKB / 16;                         // 16-byte chunks per row
    static constexpr int RPB = 64 / CH;                         // rows per 1 KiB wave load
    static constexpr int NBLK = (TN + TM) / RPB;                // wave loads per step
    static constexpr int Q = NBLK / NW;                         // loads per wave per step
    static constexpr int STAGE = (TN + TM) * BKB;               // LDS bytes per stage
    static_assert(BKB == 64 || BKB == 128, "K step");
    static_assert(TN % WN == 0 && TM % WM == 0 && WN % 16 == 0 && WM % 16 == 0, "tile shape");
    static_assert(NBLK % NW == 0 && Q >= 1, "loader split");
    static_assert(NS >= 2 && NS * STAGE <= 160 * 1024, "LDS");
    static_assert((NS - 1) * Q < 64, "vmcnt range");
};

using TileL = Tile<256, 256, 128, 64, 2, 128>;  // 8 waves, 128 KiB
using TileG = Tile<192, 256, 96, 64, 2, 128>;   // 8 waves, 112 KiB
using TileM = Tile<128, 128, 64, 64, 4, 128>;   // 4 waves, 128 KiB
using TileS = Tile<64, 64, 32, 32, 4, 128>;     // 4 waves, 64 KiB

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

// LDS rows hold BKB bytes (CH chunks of 16).  Chunk kc of row r sits at slot
// kc ^ swz(r), swz(r) = (r / (128 / BKB)) mod CH, so the 16-byte fragment
// reads of 8 consecutive rows (one or two rows per 128 bytes) hit 8 different
// bank groups.
template <class TL>
__device__ __forceinline__ int swz(int row) {
    return TL::BKB == 128 ? (row & 7) : ((row >> 1) & 3);
}
template <class TL>
__device__ __forceinline__ int lds_at(int row, int kc) {
    return row * TL::BKB + ((kc ^ swz<TL>(row)) << 4);
}

// Global -> LDS without registers: one buffer_load_dwordx4 ... lds per wave
// fills 1 KiB of LDS = RPB rows x BKB bytes of a K step.  The LDS side of such
// a load is fixed (lane l writes bytes 16l .. 16l+15 of the KiB), so each lane
// fetches the global chunk that belongs in that slot of the swizzled layout:
// row RPB blk + l / CH, logical chunk (l mod CH) ^ swz(that row).  The blocks of
// the A (W-side) and B (x-side) tiles are numbered together and dealt to the
// waves round-robin.
template <class TL>
struct Loader {
    // The blocks of the A (W-side) and B (x-side) tiles are dealt round-robin,
    // so a wave's load q covers A block wave + q NW (q < QA) or B block
    // wave + (q - QA) NW: its lane offset is the lane's offset in the wave's
    // first block of that side plus a uniform stride.
    static constexpr int QA = TL::TN / TL::RPB / TL::NW, QB = TL::TM / TL::RPB / TL::NW;
    static_assert(QA * TL::RPB * TL::NW == TL::TN && QB * TL::RPB * TL::NW == TL::TM, "loader split");
    uint32_t va, vb;          // lane offsets in the first A / B block, k step 0
    uint32_t sa, sb;          // byte stride between a wave's consecutive blocks (uniform)
    __device__ __forceinline__ static uint32_t chunk16(int lane) {
        return (uint32_t)((lane % TL::CH) ^ swz<TL>(lane / TL::CH)) << 4;
    }
    __device__ __forceinline__ void init(uint32_t a_bytes, uint32_t b_bytes, int wave, int lane) {
        const uint32_t row = (uint32_t)(wave * TL::RPB + lane / TL::CH);
        va = row * a_bytes + chunk16(lane);
        vb = row * b_bytes + chunk16(lane);
        sa = (uint32_t)(TL::NW * TL::RPB) * a_bytes;
        sb = (uint32_t)(TL::NW * TL::RPB) * b_bytes;
    }
    // loads of one K step (kb0 = its first byte within a row) into an LDS stage;
    // rows past a tile's valid rows read zeros through the buffer range check
    // (the row offset is in the range-checked vector offset), and in the last,
    // ragged step the chunks past the row end are sent out of range too
    template <bool DO_A = true, bool DO_B = true>
    __device__ __forceinline__ void issue(char* stage, __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb,
                                          uint32_t row_bytes, uint32_t kb0, int wave, int lane) const {
        const bool ok = kb0 + TL::BKB <= row_bytes || kb0 + chunk16(lane) < row_bytes;
#pragma unroll
        for (int q = 0; q < (DO_A ? QA : 0); ++q) {
            const uint32_t v = ok ? va + (uint32_t)q * sa : OOB;
            auto* dst = (__attribute__((address_space(3))) void*)(stage + (wave + q * TL::NW) * 1024);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, dst, 16, v, (int)kb0, 0, 0);
        }
#pragma unroll
        for (int q = 0; q < (DO_B ? QB : 0); ++q) {
            const uint32_t v = ok ? vb + (uint32_t)q * sb : OOB;
            auto* dst = (__attribute__((address_space(3))) void*)(stage + (wave + (QA + q) * TL::NW) * 1024);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, dst, 16, v, (int)kb0, 0, 0);
        }
    }
};

// An operand stored with the contraction index as rows ([contraction][ld],
// 16-bit; x, dy and W in the backward): a K step is 64 contraction rows of
// ROWS consecutive columns, kept in LDS in that orientation (rows of ROWS*2
// bytes, 16-byte slot s of row r holding chunk s ^ tswz(r)) and turned into
// MFMA fragments by the transposing LDS read.  A wave load still fills 1 KiB
// (KRB whole rows), and a side still takes ROWS/8 of them per step.  The step
// advance is in the per-lane offset (rows past the matrix fall outside the
// buffer range); lanes whose columns lie past the stored row read nothing.
template <class TL, int ROWS>
struct LoaderT {
    static constexpr int CPR = ROWS / 8;                 // 16-byte chunks per LDS row
    static constexpr int KRB = 64 / CPR;                 // contraction rows per 1 KiB wave load
    uint32_t off;    // lane's byte offset in its first block at step 0 (OOB: nothing to read)
    uint32_t sa;     // byte stride between a wave's consecutive blocks
    uint32_t step;   // bytes per K step (64 rows)
    __device__ __forceinline__ void init(int64_t col0, int64_t ld, int wave, int lane) {
        // (a wave's later blocks start 16 rows on: the same permutation)
        static_assert(CPR * KRB == 64 && (TL::NW * KRB) % 16 == 0, "transposed tile");
        const int r = wave * KRB + lane / CPR;               // contraction row within the step
        const int64_t col = col0 + 8 * ((lane % CPR) ^ tswz<CPR>(r));
        off = col < ld ? (uint32_t)((r * ld + col) * 2) : OOB;
        sa = (uint32_t)(TL::NW * KRB * ld * 2);
        step = (uint32_t)(64 * ld * 2);
    }
};

// This wave's operand fragments of MFMA substep `sub` (64 bytes per row) from
// an LDS stage: FN 16-row blocks of the A tile, FM of the B tile.
template <class TL, bool TA = false, bool TB = false>
__device__ __forceinline__ void read_frags(const char* st, int sub, i32x4 (&fa)[TL::FN], i32x4 (&fb)[TL::FM],
                                           int lane, int wn, int wm) {
    const int kc = sub * 4 + (lane >> 4);
    const char* sb = st + TL::TN * TL::BKB;
#pragma unroll
    for (int i = 0; i < TL::FN; ++i) {
        if constexpr (TA) fa[i] = frag_t<TL::TN>(st, sub * 32, wn * TL::WN + i * 16, lane);
        else fa[i] = *(const i32x4*)(st + lds_at<TL>(wn * TL::WN + i * 16 + (lane & 15), kc));
    }
#pragma unroll
    for (int j = 0; j < TL::FM; ++j) {
        if constexpr (TB) fb[j] = frag_t<TL::TM>(sb, sub * 32, wm * TL::WM + j * 16, lane);
        else fb[j] = *(const i32x4*)(sb + lds_at<TL>(wm * TL::WM + j * 16 + (lane & 15), kc));
    }
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
// B = h_r), then the main steps over K (A = W_c, B = x_c).  Steps at or past
// KT are issued too, entirely out of range: they write zeros into a stage that
// is never read again, so every pipeline step issues exactly Q loads per wave
// and the vmcnt bookkeeping needs no branches.
template <class TL, bool TA = false, bool TB = false>
struct Steps {
    Loader<TL> lf, lm;
    LoaderT<TL, TL::TN> tma;         // transposed A side (main steps; no fold)
    LoaderT<TL, TL::TM> tmb;         // transposed B side
    const char *tma_p, *tmb_p;
    uint32_t tma_n, tmb_n;           // whole-matrix byte extents
    const char *fa, *fb, *ma, *mb;   // operand rows of this tile
    uint32_t nfa, nfb, nma, nmb;     // their byte extents (buffer range)
    uint32_t fbytes, kbytes;
    int RF, KT;
    int k0;                          // first main step of this workgroup's K split
    __device__ __forceinline__ void issue(char* smem, int s, int wave, int lane) const {
        char* st = smem + (s % TL::NS) * TL::STAGE;
        const bool fold = s < RF;
        // select plain values, then build the resources (a conditional over
        // the resource type itself loses the kernel's host stub)
        const auto ra = make_rsrc(fold ? fa : ma, fold ? nfa : nma);
        const auto rb = make_rsrc(fold ? fb : mb, fold ? nfb : nmb);
        Loader<TL> l;
        l.va = fold ? lf.va : lm.va;
        l.vb = fold ? lf.vb : lm.vb;
        l.sa = fold ? lf.sa : lm.sa;
        l.sb = fold ? lf.sb : lm.sb;
        const uint32_t row_bytes = s < KT ? (fold ? fbytes : kbytes) : 0u;   // 0: all out of range
        const uint32_t sidx = (uint32_t)(fold ? s : s - RF + k0);          // step within the fold / main
        l.template issue<!TA, !TB>(st, ra, rb, row_bytes, sidx * TL::BKB, wave, lane);
        if constexpr (TA) {
            const auto rt = make_rsrc(tma_p, tma_n);
            const uint32_t adv = sidx * tma.step;
#pragma unroll
            for (int q = 0; q < Loader<TL>::QA; ++q) {
                const uint32_t v = (s < KT && tma.off != OOB) ? tma.off + (uint32_t)q * tma.sa + adv : OOB;
                auto* dst = (__attribute__((address_space(3))) void*)(st + (wave + q * TL::NW) * 1024);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rt, dst, 16, v, 0, 0, 0);
            }
        }
        if constexpr (TB) {
            const auto rt = make_rsrc(tmb_p, tmb_n);
            const uint32_t adv = sidx * tmb.step;
#pragma unroll
            for (int q = 0; q < Loader<TL>::QB; ++q) {
                const uint32_t v = (s < KT && tmb.off != OOB) ? tmb.off + (uint32_t)q * tmb.sa + adv : OOB;
                auto* dst =
                    (__attribute__((address_space(3))) void*)(st + (wave + (Loader<TL>::QA + q) * TL::NW) * 1024);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rt, dst, 16, v, 0, 0, 0);
            }
        }
    }
};

// MFMAs of one substep with NV global loads and ND LDS reads (issued just
// before, for later steps) spread between them: the matrix pipe never waits
// for a burst of memory instructions to issue.
template <class CT, class TL, int NV, int ND>
__device__ __forceinline__ void mma_spread(const i32x4 (&fa)[TL::FN], const i32x4 (&fb)[TL::FM],
                                           f32x4 (&acc)[TL::FN][TL::FM]) {
    mma<CT, TL>(fa, fb, acc);
    constexpr int G = NV > ND ? NV : ND;
    constexpr int PER = TL::FN * TL::FM / (G + 1);
#pragma unroll
    for (int g = 0; g < G; ++g) {
        if (g < NV) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // VMEM read
        if (g < ND) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
        __builtin_amdgcn_sched_group_barrier(0x008, PER, 0);             // MFMA
    }
    __builtin_amdgcn_sched_group_barrier(0x008, TL::FN * TL::FM - G * PER, 0);
}

// One K step kt (two MFMA substeps of 32 k).  On entry the fragments of its
// substep 0 are in (f0a, f0b) and steps up to kt+NS-1 have been issued.
//   substep 0: read substep 1 into (f1a, f1b); MFMAs on (f0a, f0b)
//   substep 1: wait until step kt+1 has landed (NS-2 steps after it may still be
//              in flight), barrier, refill the stage of step kt with step
//              kt+NS, read step kt+1's substep 0 into (f0a, f0b); MFMAs on (f1a, f1b)
template <class CT, class TL, bool TA = false, bool TB = false>
__device__ __forceinline__ void k_step(const Steps<TL, TA, TB>& S, char* smem, int kt, i32x4 (&f0a)[TL::FN],
                                       i32x4 (&f0b)[TL::FM], i32x4 (&f1a)[TL::FN], i32x4 (&f1b)[TL::FM],
                                       f32x4 (&acc)[TL::FN][TL::FM], int wave, int lane, int wn, int wm) {
    static_assert(TL::SUB == 2, "two substeps per K step");
    constexpr int ND = (TA ? 2 : 1) * TL::FN + (TB ? 2 : 1) * TL::FM;   // LDS reads per substep
    __builtin_amdgcn_s_waitcnt(0xC07F);   // substep 0's fragments have landed
    read_frags<TL, TA, TB>(smem + (kt % TL::NS) * TL::STAGE, 1, f1a, f1b, lane, wn, wm);
    mma_spread<CT, TL, 0, ND>(f0a, f0b, acc);
    // every MFMA of substep 0 is issued before this wave waits on memory
    __builtin_amdgcn_sched_barrier(0);

    wait_vm<(TL::NS - 2) * TL::Q>();
    lds_barrier();
    S.issue(smem, kt + TL::NS, wave, lane);
    // (past the last step this reads a stage that is never used: in bounds)
    read_frags<TL, TA, TB>(smem + ((kt + 1) % TL::NS) * TL::STAGE, 0, f0a, f0b, lane, wn, wm);
    mma_spread<CT, TL, TL::Q, ND>(f1a, f1b, acc);
}

// One main K step (operands as the forward stores them) with its memory work
// interleaved by hand.  Substep 1's MFMAs are cut into G groups of FN/G
// A-side blocks.  The first group is issued before the wait and the barrier
// (it needs only registers, so the matrix pipe has work while the waves
// meet); the loads of step kt+NS and the fragment reads of step kt+1 then go
// between the remaining groups, fenced by scheduling barriers.  (Left to the
// scheduler, the eight loads were issued back to back after the barrier with
// the matrix pipe idle: the GEMM took 4-5% longer.)
template <class CT, class TL>
__device__ __forceinline__ void k_step_main(const Steps<TL>& S, __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb,
                                            char* smem, int kt, i32x4 (&f0a)[TL::FN], i32x4 (&f0b)[TL::FM],
                                            i32x4 (&f1a)[TL::FN], i32x4 (&f1b)[TL::FM], f32x4 (&acc)[TL::FN][TL::FM],
                                            int wave, int lane, int wn, int wm) {
    constexpr int ND = TL::FN + TL::FM;
    constexpr int G = TL::FN % 4 == 0 ? 4 : (TL::FN % 3 == 0 ? 3 : 2), FNG = TL::FN / G;
    static_assert(TL::FN % G == 0, "MFMA groups");
    using LD = Loader<TL>;
    __builtin_amdgcn_s_waitcnt(0xC07F);
    read_frags<TL>(smem + (kt % TL::NS) * TL::STAGE, 1, f1a, f1b, lane, wn, wm);
    mma_spread<CT, TL, 0, ND>(f0a, f0b, acc);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0xC07F);
#pragma unroll
    for (int i = 0; i < FNG; ++i)
#pragma unroll
        for (int j = 0; j < TL::FM; ++j) acc[i][j] = CT::step(f1a[i], f1b[j], acc[i][j]);
    __builtin_amdgcn_sched_barrier(0);
    wait_vm<(TL::NS - 2) * TL::Q>();
    lds_barrier();
    // step kt+NS into the stage just consumed (out of range past the end)
    const int s = kt + TL::NS;
    char* st = smem + (s % TL::NS) * TL::STAGE;
    const uint32_t row_bytes = s < S.KT ? S.kbytes : 0u;
    const uint32_t kb0 = (uint32_t)(s - S.RF + S.k0) * TL::BKB;
    const bool ok = kb0 + TL::BKB <= row_bytes || kb0 + LD::chunk16(lane) < row_bytes;
    const char* nx = smem + ((kt + 1) % TL::NS) * TL::STAGE;
    const int kc = lane >> 4;
#pragma unroll
    for (int g = 1; g < G; ++g) {
        // loads: the A side with groups 1-2, the B side with group 3 (and the rest)
#pragma unroll
        for (int q = 0; q < LD::QA + LD::QB; ++q) {
            const int grp = 1 + (q * (G - 1)) / (LD::QA + LD::QB);
            if (grp != g) continue;
            if (q < LD::QA) {
                const uint32_t v = ok ? S.lm.va + (uint32_t)q * S.lm.sa : OOB;
                auto* dst = (__attribute__((address_space(3))) void*)(st + (wave + q * TL::NW) * 1024);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, dst, 16, v, (int)kb0, 0, 0);
            } else {
                const int qb = q - LD::QA;
                const uint32_t v = ok ? S.lm.vb + (uint32_t)qb * S.lm.sb : OOB;
                auto* dst = (__attribute__((address_space(3))) void*)(st + (wave + q * TL::NW) * 1024);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, dst, 16, v, (int)kb0, 0, 0);
            }
        }
        // fragment reads of step kt+1, substep 0 (spread over the groups)
#pragma unroll
        for (int i = 0; i < TL::FN; ++i)
            if (i * (G - 1) / TL::FN + 1 == g)
                f0a[i] = *(const i32x4*)(nx + lds_at<TL>(wn * TL::WN + i * 16 + (lane & 15), kc));
#pragma unroll
        for (int j = 0; j < TL::FM; ++j)
            if (j * (G - 1) / TL::FM + 1 == g)
                f0b[j] = *(const i32x4*)(nx + TL::TN * TL::BKB + lds_at<TL>(wm * TL::WM + j * 16 + (lane & 15), kc));
#pragma unroll
        for (int i = g * FNG; i < (g + 1) * FNG; ++i)
#pragma unroll
            for (int j = 0; j < TL::FM; ++j) acc[i][j] = CT::step(f1a[i], f1b[j], acc[i][j]);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// The output tile through LDS, so that every store writes whole rows of it.
// A lane's MFMA results are 4 consecutive n of one token row m for each 16x16
// block, so a store straight from them covers 16 rows x 8-16 bytes: at the
// bf16 16384 x 8192 x 8192 size those partial-line stores took ~9 us at the
// end of each tile.  Here the waves write their blocks (scaled, biased,
// rounded to y's dtype) into the free pipeline stages as rows of the tile
// (16-byte chunk c of row r at slot c ^ (r & 7)), and then store 16-byte
// chunks in row order: a wave's store covers 1 KiB of consecutive rows.  A
// tile larger than the stages (fp32 output of the 256-row tiles) goes in two
// passes of half its rows.  Needs N * ES a multiple of 16 and y 16-byte
// aligned (a chunk is then all inside y's row or all past its end).
template <class TL, int ES, bool GAIN>
__device__ __forceinline__ void epilogue_rows(const GemmParams& p, char* smem, const f32x4 (&acc)[TL::FN][TL::FM],
                                              const float* biasv, const float* gainv, int64_t n0, int64_t m0,
                                              int wave, int lane, int wn, int wm) {
    constexpr int RB = TL::TN * ES, CHR = RB / 16;   // bytes and 16-byte chunks of a tile row
    constexpr int CAP = TL::NS * TL::STAGE;
    constexpr int TMP = TL::TM * RB <= CAP ? TL::TM : TL::TM / 2;   // rows per pass
    constexpr int PASSES = TL::TM / TMP, IT = TMP * CHR / (TL::NW * 64);
    static_assert(TMP * RB <= CAP && TL::TM % TMP == 0 && TMP % TL::WM == 0 && CHR % 8 == 0, "staged rows");
    static_assert(IT * TL::NW * 64 == TMP * CHR, "whole wave stores");
    const int64_t yrow = p.N * ES;
    // (the barriers fence the scheduler, and the stores go four chunks at a
    // time: with two passes the second pass's writers still hold their
    // accumulators during the first pass's stores, and a deeper batch, or
    // outputs computed ahead of a barrier, made the registers spill)
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
        __syncthreads();   // the stages (then the previous pass's rows) are free
        __builtin_amdgcn_sched_barrier(0);
        if ((wm * TL::WM) / TMP == ps) {
#pragma unroll
            for (int i = 0; i < TL::FN; ++i) {
                const int nl = wn * TL::WN + i * 16 + 4 * (lane >> 4);
                const float* bias = biasv + 4 * i;
                const float* gain = gainv + (GAIN ? 4 * i : 0);
#pragma unroll
                for (int j = 0; j < TL::FM; ++j) {
                    const int r = wm * TL::WM + j * 16 + (lane & 15) - ps * TMP;
                    float v[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = acc[i][j][e] * (GAIN ? gain[e] : p.post) + bias[e];
                    const int cb = nl * ES;   // byte column
                    char* dst = smem + r * RB + ((((cb >> 4) ^ (r & 7)) << 4) | (cb & 15));
                    if constexpr (ES == 4) {
                        *(f32x4*)dst = f32x4{v[0], v[1], v[2], v[3]};
                    } else {
                        const uint32_t lo = p.y_dt == DT_F16 ? pack_f16x2(v[0], v[1]) : pack_bf16x2(v[0], v[1]);
                        const uint32_t hi = p.y_dt == DT_F16 ? pack_f16x2(v[2], v[3]) : pack_bf16x2(v[2], v[3]);
                        *(i32x2*)dst = i32x2{(int)lo, (int)hi};
                    }
                }
            }
        }
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll 4
        for (int it = 0; it < IT; ++it) {
            const int idx = (it * TL::NW + wave) * 64 + lane;
            const int r = idx / CHR, c = idx % CHR;
            const i32x4 d = *(const i32x4*)(smem + r * RB + ((c ^ (r & 7)) << 4));
            const int64_t m = m0 + ps * TMP + r, n = n0 + c * (16 / ES);
            if (m < p.M && n < p.N) *(i32x4*)((char*)p.y + m * yrow + n * ES) = d;
        }
    }
}

// GAIN: a per-output-feature factor gain[n] in place of post (an instance of
// its own, so the others carry no registers for it)
// TA / TB: the A / B operand stored with the contraction index as rows
// (LoaderT; main steps only, launched with both and no fold); otherwise
// operands as the forward stores them.
// ROWS: the outputs go out through LDS as whole rows (epilogue_rows; no K
// split, N * bytes of y's dtype a multiple of 16, y 16-byte aligned): an
// instance of its own, since both epilogues in one kernel made it spill.
template <class CT, class TL, bool GAIN, bool TA = false, bool TB = false, bool ROWS = false>
__global__ __launch_bounds__(TL::NT, 1) void gemm_kernel(GemmParams p, int tiles_n, int tiles_m, int group_m) {
    // the operand stages, then the tile's bias widened to fp32.  One LDS
    // object: with a second __shared__ array the compiler could no longer
    // tell the direct-to-LDS loads from the fragment reads and waited for
    // every load right after issuing it.
    __shared__ __attribute__((aligned(16))) char smem[TL::NS * TL::STAGE + TL::TN * 4];
    float* sbias = (float*)(smem + TL::NS * TL::STAGE);
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
    Steps<TL, TA, TB> S;
    S.fbytes = (uint32_t)(p.rf * CT::es);
    S.kbytes = (uint32_t)(p.K * CT::es);
    // K split (blockIdx.y of gridDim.y): a contiguous range of the main steps;
    // the fold steps go with split 0
    const int KM = (int)((S.kbytes + TL::BKB - 1) / TL::BKB);
    const int per = (KM + (int)gridDim.y - 1) / (int)gridDim.y;
    S.k0 = (int)blockIdx.y * per;
    const int nmain = KM - S.k0 < per ? (KM - S.k0 > 0 ? KM - S.k0 : 0) : per;
    S.RF = blockIdx.y == 0 ? (int)((S.fbytes + TL::BKB - 1) / TL::BKB) : 0;
    S.KT = S.RF + nmain;
    S.fa = (const char*)p.af + n0 * S.fbytes;
    S.fb = (const char*)p.bf + m0 * S.fbytes;
    S.ma = (const char*)p.a + n0 * S.kbytes;
    S.mb = (const char*)p.b + m0 * S.kbytes;
    S.nfa = (uint32_t)rows_a * S.fbytes;
    S.nfb = (uint32_t)rows_b * S.fbytes;
    S.nma = (uint32_t)rows_a * S.kbytes;
    S.nmb = (uint32_t)rows_b * S.kbytes;
    S.lf.init(S.fbytes, S.fbytes, wave, lane);
    S.lm.init(S.kbytes, S.kbytes, wave, lane);
    if constexpr (TA) {
        S.tma.init(n0, p.lda_t, wave, lane);
        S.tma_p = (const char*)p.a;
        S.tma_n = (uint32_t)(p.K * p.lda_t * 2);
    }
    if constexpr (TB) {
        S.tmb.init(m0, p.ldb_t, wave, lane);
        S.tmb_p = (const char*)p.b;
        S.tmb_n = (uint32_t)(p.K * p.ldb_t * 2);
    }
    const int KT = S.KT;
    // the tile's bias, loaded before the first operand loads (so it lands
    // first) and written to LDS after them; the epilogue reads it from there
    float bv = 0.f;
    if (p.bias != nullptr && p.ksplit <= 1 && tid < TL::TN)
        bv = n0 + tid < p.N ? load_as_f32(p.bias, p.bias_dt, n0 + tid) : 0.f;
    if (KT > 0) {
        i32x4 f0a[FN], f0b[FM], f1a[FN], f1b[FM];
        // steps 0 .. NS-1 fill every stage; step 0 must land (NS-1 steps follow it)
#pragma unroll
        for (int s0 = 0; s0 < TL::NS; ++s0) S.issue(smem, s0, wave, lane);
        wait_vm<(TL::NS - 1) * TL::Q>();
        lds_barrier();
        if (tid < TL::TN) sbias[tid] = bv;
        read_frags<TL, TA, TB>(smem, 0, f0a, f0b, lane, wn, wm);
        // fold steps, then acc = scale * (h_r . up_c^T) once, then the main steps:
        // the accumulators see no vector ALU work inside either loop
        for (int kt = 0; kt < S.RF; ++kt) k_step<CT, TL, TA, TB>(S, smem, kt, f0a, f0b, f1a, f1b, acc, wave, lane, wn, wm);
        if (S.RF > 0) {
#pragma unroll
            for (int i = 0; i < FN; ++i)
#pragma unroll
                for (int j = 0; j < FM; ++j) acc[i][j] *= p.scale;
        }
        if constexpr (!TA && !TB) {
            const auto ra = make_rsrc(S.ma, S.nma);
            const auto rb = make_rsrc(S.mb, S.nmb);
            for (int kt = S.RF; kt < KT; ++kt)
                k_step_main<CT, TL>(S, ra, rb, smem, kt, f0a, f0b, f1a, f1b, acc, wave, lane, wn, wm);
        } else {
            for (int kt = S.RF; kt < KT; ++kt)
                k_step<CT, TL, TA, TB>(S, smem, kt, f0a, f0b, f1a, f1b, acc, wave, lane, wn, wm);
        }
        wait_vm<0>();   // the out-of-range loads past the last step still write LDS
    } else if (tid < TL::TN) {
        sbias[tid] = bv;
    }

    // 3. epilogue: lane holds, per 16x16 block, 4 consecutive n for one m.
    if (p.ksplit > 1) {
        // this split's fp32 sums; the reduction adds the bias and rounds
        float* part = p.partial + (int64_t)blockIdx.y * p.M * p.N;
#pragma unroll
        for (int i = 0; i < FN; ++i) {
            const int64_t nb = n0 + wn * TL::WN + i * 16 + 4 * (lane >> 4);
#pragma unroll
            for (int j = 0; j < FM; ++j) {
                const int64_t m = m0 + wm * TL::WM + j * 16 + (lane & 15);
                if (m >= p.M) continue;
                float* dst = part + m * p.N + nb;
                if (p.vec_store && nb + 3 < p.N) {
                    *(f32x4*)dst = acc[i][j];
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (nb + e < p.N) dst[e] = acc[i][j][e];
                }
            }
        }
        return;
    }
    //    The bias of every block comes from LDS (a per-feature gain from global
    //    memory), all before the first store.
    float biasv[FN * 4] = {};
    if (p.bias != nullptr) {
        __syncthreads();
#pragma unroll
        for (int i = 0; i < FN; ++i) {
            const f32x4 b4 = *(const f32x4*)(sbias + wn * TL::WN + i * 16 + 4 * (lane >> 4));
            biasv[4 * i] = b4[0]; biasv[4 * i + 1] = b4[1]; biasv[4 * i + 2] = b4[2]; biasv[4 * i + 3] = b4[3];
        }
    }
    float gainv[GAIN ? FN * 4 : 1];
    if constexpr (GAIN) {
        int64_t idx[FN * 4];
#pragma unroll
        for (int i = 0; i < FN * 4; ++i) idx[i] = n0 + wn * TL::WN + (i >> 2) * 16 + 4 * (lane >> 4) + (i & 3);
        load_n_as_f32<FN * 4>(p.gain, DT_F32, idx, p.N, gainv);
    }
    if constexpr (ROWS) {
        if (p.y_dt == DT_F32) epilogue_rows<TL, 4, GAIN>(p, smem, acc, biasv, gainv, n0, m0, wave, lane, wn, wm);
        else epilogue_rows<TL, 2, GAIN>(p, smem, acc, biasv, gainv, n0, m0, wave, lane, wn, wm);
        return;
    }
#pragma unroll
    for (int i = 0; i < FN; ++i) {
        const int64_t nb = n0 + wn * TL::WN + i * 16 + 4 * (lane >> 4);
        const float* bias = biasv + 4 * i;
        const float* gain = gainv + (GAIN ? 4 * i : 0);
#pragma unroll
        for (int j = 0; j < FM; ++j) {
            const int64_t m = m0 + wm * TL::WM + j * 16 + (lane & 15);
            if (m >= p.M) continue;
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float a = acc[i][j][e];
                v[e] = a * (GAIN ? gain[e] : p.post) + bias[e];
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
                const uint32_t lo = p.y_dt == DT_F16 ? pack_f16x2(v[0], v[1]) : pack_bf16x2(v[0], v[1]);
                const uint32_t hi = p.y_dt == DT_F16 ? pack_f16x2(v[2], v[3]) : pack_bf16x2(v[2], v[3]);
                const uint16_t o[4] = {(uint16_t)lo, (uint16_t)(lo >> 16), (uint16_t)hi, (uint16_t)(hi >> 16)};
                uint16_t* y = (uint16_t*)p.y;
                if (p.vec_store && nb + 3 < p.N) {
                    *(i32x2*)(y + base) = i32x2{(int)lo, (int)hi};
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (nb + e < p.N) y[base + e] = o[e];
                }
            }
        }
    }
}

// y = round_out(gain or post * (sum of the K splits' partial sums, in split order) + b)
__global__ __launch_bounds__(256) void gemm_reduce_kernel(GemmParams p) {
    const int64_t MN = p.M * p.N;
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < MN; i += stride) {
        float v = p.partial[i];
        for (int k = 1; k < p.ksplit; ++k) v += p.partial[(int64_t)k * MN + i];
        const int64_t n = i % p.N;
        v *= p.gain != nullptr ? p.gain[n] : p.post;
        if (p.bias != nullptr) v += load_as_f32(p.bias, p.bias_dt, n);
        if (p.y_dt == DT_F32) ((float*)p.y)[i] = v;
        else ((uint16_t*)p.y)[i] = p.y_dt == DT_F16 ? f32_to_f16(v) : f32_to_bf16(v);
    }
}

template <class CT, class TL>
static hipError_t run(const GemmParams& p, hipStream_t s) {
    const int tiles_n = (int)((p.N + TL::TN - 1) / TL::TN);
    const int tiles_m = (int)((p.M + TL::TM - 1) / TL::TM);
    const int nblk = tiles_n * tiles_m;
    const int ks = p.ksplit > 1 ? p.ksplit : 1;
    // (a K split applies the gain in its reduction)
    if constexpr (CT::dt != DT_F32 && TL::TN != 192) {
        if (p.ta && p.tb)
            hipLaunchKernelGGL((gemm_kernel<CT, TL, false, true, true>), dim3(nblk, ks), dim3(TL::NT), 0, s, p, tiles_n,
                               tiles_m, 4);
    }
    // whole-row stores of the output (epilogue_rows)
    const bool rows = ks == 1 && (p.N * (p.y_dt == DT_F32 ? 4 : 2)) % 16 == 0 && ((uintptr_t)p.y & 15) == 0;
    if (p.ta || p.tb) {
        // (no transposed instance for fp32 compute or the 192-row tile: refused above)
    } else if (p.gain != nullptr && ks == 1) {
        if (rows)
            hipLaunchKernelGGL((gemm_kernel<CT, TL, true, false, false, true>), dim3(nblk, ks), dim3(TL::NT), 0, s, p,
                               tiles_n, tiles_m, 4);
        else
            hipLaunchKernelGGL((gemm_kernel<CT, TL, true>), dim3(nblk, ks), dim3(TL::NT), 0, s, p, tiles_n, tiles_m, 4);
    } else if (rows) {
        hipLaunchKernelGGL((gemm_kernel<CT, TL, false, false, false, true>), dim3(nblk, ks), dim3(TL::NT), 0, s, p,
                           tiles_n, tiles_m, 4);
    } else {
        hipLaunchKernelGGL((gemm_kernel<CT, TL, false>), dim3(nblk, ks), dim3(TL::NT), 0, s, p, tiles_n, tiles_m, 4);
    }
    if (ks > 1) {
        const int64_t blocks = (p.M * p.N + 255) / 256;
        hipLaunchKernelGGL(gemm_reduce_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, s, p);
    }
    return hipGetLastError();
}

// ---- the planner's device model ------------------------------------------------
// Published MI355X dense peaks per CU (256 CUs: 2.5 PFLOP/s with 16-bit
// operands, 157.3 TFLOP/s fp32) and its 8 TB/s of HBM, the defaults until the
// device's own rates are measured.
constexpr double PUB_MFMA16_PER_CU = 2500e12 / 256.0, PUB_MFMA32_PER_CU = 157.3e12 / 256.0, PUB_HBM = 8.0e12;

static std::mutex rates_mu;
static std::map<int, DeviceRates> rates_by_dev;

DeviceRates device_rates() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return DeviceRates{256, 256 * PUB_MFMA16_PER_CU, 256 * PUB_MFMA32_PER_CU, PUB_HBM, 0};
    }
    std::lock_guard<std::mutex> lk(rates_mu);
    auto it = rates_by_dev.find(dev);
    if (it != rates_by_dev.end()) return it->second;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
        (void)hipGetLastError();
        cus = 256;
    }
    const DeviceRates r{cus, cus * PUB_MFMA16_PER_CU, cus * PUB_MFMA32_PER_CU, PUB_HBM, 0};
    rates_by_dev[dev] = r;
    return r;
}

// Dense MFMA issue: every wave runs 8 independent accumulator chains of its
// compute type's step on operands of 1.0 (`one`: the pattern of 1.0 in each
// element; exact sums, no special values).
// (The VGPR budget makes the compiler keep the chains in VGPRs, in the
// MFMA's VGPR form; with accumulation registers it copied the 16-bit chains
// through VGPRs every iteration.)
template <class CT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_num_vgpr(128))) void mfma_rate_kernel(f32x4* out, int iters,
                                                                                          uint32_t one) {
    const i32x4 a = i32x4{(int)one, (int)one, (int)one, (int)one};
    f32x4 acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] = CT::step(a, a, acc[c]);
    }
    // every chain is stored, so none is dropped
#pragma unroll
    for (int c = 0; c < 8; ++c) out[((size_t)blockIdx.x * 256 + threadIdx.x) * 8 + c] = acc[c];
}

// best of three timed launches of fn on s, in seconds
template <class F>
static hipError_t best_of_3(hipStream_t s, hipEvent_t a, hipEvent_t b, F fn, double* sec) {
    double best = 1e300;
    hipError_t e = fn();   // warm-up
    for (int rep = 0; rep < 3 && e == hipSuccess; ++rep) {
        float ms = 0.f;
        if ((e = hipEventRecord(a, s)) != hipSuccess) break;
        if ((e = fn()) != hipSuccess) break;
        if ((e = hipEventRecord(b, s)) != hipSuccess || (e = hipEventSynchronize(b)) != hipSuccess ||
            (e = hipEventElapsedTime(&ms, a, b)) != hipSuccess)
            break;
        best = std::min(best, (double)ms * 1e-3);
    }
    *sec = best;
    return e;
}

hipError_t measure_device_rates(hipStream_t s) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    DeviceRates r = device_rates();
    constexpr size_t COPY = 256u << 20;
    constexpr int ITERS = 2048, WG_PER_CU = 4;   // 16 waves per CU
    const unsigned grid = (unsigned)(r.cus * WG_PER_CU);
    // the rate kernels' outputs (8 vectors per thread) reuse the copy's buffer
    if ((size_t)grid * 256 * 8 * sizeof(f32x4) > 2 * COPY) return hipErrorInvalidValue;
    char* buf = nullptr;
    hipEvent_t a = nullptr, b = nullptr;
    if ((e = hipMalloc(&buf, 2 * COPY)) != hipSuccess) return e;
    if ((e = hipEventCreate(&a)) == hipSuccess && (e = hipEventCreate(&b)) == hipSuccess) {
        double t_copy = 0, t16 = 0, t32 = 0;
        e = best_of_3(s, a, b, [&] { return hipMemcpyAsync(buf + COPY, buf, COPY, hipMemcpyDeviceToDevice, s); },
                      &t_copy);
        f32x4* out = (f32x4*)buf;   // grid * 256 * 8 vectors: 32 MiB at 256 CUs
        if (e == hipSuccess)
            e = best_of_3(s, a, b, [&] {
                hipLaunchKernelGGL(mfma_rate_kernel<CF16>, dim3(grid), dim3(256), 0, s, out, ITERS, 0x3C003C00u);
                return hipGetLastError();
            }, &t16);
        if (e == hipSuccess)
            e = best_of_3(s, a, b, [&] {
                hipLaunchKernelGGL(mfma_rate_kernel<CF32>, dim3(grid), dim3(256), 0, s, out, ITERS / 4, 0x3F800000u);
                return hipGetLastError();
            }, &t32);
        if (e == hipSuccess && t_copy > 0 && t16 > 0 && t32 > 0) {
            const double waves = (double)grid * 4.0;
            r.hbm = 2.0 * (double)COPY / t_copy;                                  // read + write
            r.mfma16 = waves * ITERS * 8.0 * (2.0 * 16 * 16 * 32) / t16;           // 16x16x32 steps
            r.mfma32 = waves * (ITERS / 4) * 8.0 * 4.0 * (2.0 * 16 * 16 * 4) / t32;   // 4 x 16x16x4 per step
            r.measured = 1;
            std::lock_guard<std::mutex> lk(rates_mu);
            rates_by_dev[dev] = r;
        }
    }
    if (a) (void)hipEventDestroy(a);
    if (b) (void)hipEventDestroy(b);
    const hipError_t ef = hipFree(buf);
    return e != hipSuccess ? e : ef;
}

// Tile choice: fewest "rounds" of workgroups over the device's CUs, weighted
// by tile area and a per-shape efficiency penalty (smaller tiles re-read more).
enum { T_L, T_G, T_M, T_S };
static int pick_tile(int64_t M, int64_t N, bool f32) {
    struct C { int id, tn, tm; double pen; };
    const C cands16[] = {{T_L, 256, 256, 1.0}, {T_G, 192, 256, 1.0}, {T_M, 128, 128, 1.3}, {T_S, 64, 64, 2.0}};
    const C cands32[] = {{T_M, 128, 128, 1.0}, {T_S, 64, 64, 1.5}};
    const C* c = f32 ? cands32 : cands16;
    const int nc = f32 ? 2 : 4;
    int best = c[0].id;
    double best_cost = 1e300;
    const double cus = (double)device_rates().cus;
    for (int i = 0; i < nc; ++i) {
        const double tiles = (double)((N + c[i].tn - 1) / c[i].tn) * (double)((M + c[i].tm - 1) / c[i].tm);
        const double rounds = std::ceil(tiles / cus);
        const double cost = rounds * c[i].tn * c[i].tm * c[i].pen;
        if (cost < best_cost) { best_cost = cost; best = c[i].id; }
    }
    return best;
}

// The fp32 partial sums of a K split ([ksplit][M][N]) stay below this: splits
// pay off only where few output tiles leave CUs idle, i.e. at small M * N.
constexpr double KSPLIT_PARTIAL_MAX = 32.0 * 1024 * 1024;

int gemm_ksplit(int64_t M, int64_t N, int64_t K, int c_dt) {
    int tn, tm;
    gemm_tile_shape(M, N, c_dt, &tn, &tm);
    const int64_t tiles = ((N + tn - 1) / tn) * ((M + tm - 1) / tm);
    const int64_t ksteps = (K * (c_dt == DT_F32 ? 4 : 2) + 127) / 128;
    const int64_t cus = device_rates().cus;
    if (tiles >= cus / 2 || tiles == 0) return 1;
    // about one workgroup per CU, at least 4 K steps each, at most 8 splits
    int64_t ks = cus / tiles;
    if (ks > ksteps / 4) ks = ksteps / 4;
    if (ks > 8) ks = 8;
    while (ks > 1 && (double)M * (double)N * 4.0 * (double)ks > KSPLIT_PARTIAL_MAX) --ks;
    return ks > 1 ? (int)ks : 1;
}

// A contraction over the tokens read in place (the backward's dDown and dUp:
// an M x N output with one side the rank, K the token count): the output tile
// covers the rank side whole, so that the token-major operand (x or dy, the
// large one) streams through once; a 64-wide tile read it twice at rank 128.
// The K split then gives about one workgroup per CU (two for the 64 x 64 tile,
// whose stages take half the LDS), at least 4 K steps each, at most 8 splits.
int gemm_tok_plan(int64_t M, int64_t N, int64_t K, int* tile) {
    const int64_t r = M < N ? M : N;
    const int t = r <= 64 ? T_S : (r <= 128 ? T_M : T_L);
    int tn, tm;
    gemm_tile_dims(t, &tn, &tm);
    *tile = t;
    const int64_t tiles = ((N + tn - 1) / tn) * ((M + tm - 1) / tm);
    const int64_t ksteps = (K * 2 + 127) / 128;
    if (tiles == 0) return 1;
    const int64_t want = device_rates().cus * (t == T_S ? 2 : 1);
    int64_t ks = (want + tiles - 1) / tiles;
    if (ks > ksteps / 4) ks = ksteps / 4;
    if (ks > 8) ks = 8;
    return ks > 1 ? (int)ks : 1;
}

void gemm_tile_shape(int64_t M, int64_t N, int c_dt, int* tn, int* tm) {
    static const int shape[4][2] = {{256, 256}, {192, 256}, {128, 128}, {64, 64}};
    const int t = pick_tile(M, N, c_dt == DT_F32);
    *tn = shape[t][0];
    *tm = shape[t][1];
}

void gemm_tile_dims(int tile, int* tn, int* tm) {
    static const int shape[4][2] = {{256, 256}, {192, 256}, {128, 128}, {64, 64}};
    const int t = tile < 0 || tile > 3 ? 3 : tile;
    *tn = shape[t][0];
    *tm = shape[t][1];
}

// The cost model: every workgroup of a tile runs its share of the K steps on
// one CU (one workgroup per CU for every tile) at the device's MFMA rate per
// CU; that rate falls with the tile's operand re-reads (the penalties of
// pick_tile); a K split adds the fp32 partial sums' round trip through HBM at
// the device's rate and a second launch.  The set of candidates does not
// depend on the rates, only their order does.
static bool plan_candidate(int64_t M, int64_t N, int64_t K, int tile, int ks, int c_dt) {
    if (ks == 1) return true;
    int tn, tm;
    gemm_tile_dims(tile, &tn, &tm);
    const int64_t tiles = ((N + tn - 1) / tn) * ((M + tm - 1) / tm);
    const int64_t ksteps = (K * (c_dt == DT_F32 ? 4 : 2) + 127) / 128;
    return tiles < device_rates().cus && ks <= ksteps / 4 && (double)M * (double)N * 4.0 * (double)ks <= KSPLIT_PARTIAL_MAX;
}

int gemm_plan_ksplit_max(int64_t M, int64_t N, int64_t K, int c_dt) {
    int ks_max = gemm_ksplit(M, N, K, c_dt);
    const bool f32 = c_dt == DT_F32;
    const int tiles16[] = {T_L, T_G, T_M, T_S}, tiles32[] = {T_M, T_S};
    for (int i = 0; i < (f32 ? 2 : 4); ++i)
        for (int ks = 2; ks <= 8; ks *= 2)
            if (plan_candidate(M, N, K, f32 ? tiles32[i] : tiles16[i], ks, c_dt)) ks_max = std::max(ks_max, ks);
    return ks_max;
}

int gemm_plan(int64_t M, int64_t N, int64_t K, int64_t rf, int c_dt, GemmCand* out, int max_out) {
    if (max_out <= 0) return 0;
    const bool f32 = c_dt == DT_F32;
    const double es = f32 ? 4.0 : 2.0;
    const DeviceRates dr = device_rates();
    const double cus = (double)dr.cus;
    const double cu_rate = (f32 ? dr.mfma32 : dr.mfma16) / cus;   // flop/s per CU
    const double hbm = dr.hbm;
    struct T { int id; double pen; };
    const T t16[] = {{T_L, 1.0}, {T_G, 1.0}, {T_M, 1.3}, {T_S, 2.0}};
    const T t32[] = {{T_M, 1.0}, {T_S, 1.5}};
    const T* ts = f32 ? t32 : t16;
    const int nt = f32 ? 2 : 4;
    const int64_t ksteps = (int64_t)((K * es + 127) / 128);
    auto cost = [&](int tile, int ks, double pen) {
        int tn, tm;
        gemm_tile_dims(tile, &tn, &tm);
        const double tiles = (double)((N + tn - 1) / tn) * (double)((M + tm - 1) / tm);
        const double rounds = std::ceil(tiles * ks / cus);
        const double steps = std::ceil((double)ksteps / ks) + (double)((rf * (int64_t)es + 127) / 128);
        const double step_s = 2.0 * tn * tm * (128.0 / es) / cu_rate * pen;
        double t = rounds * steps * step_s + 2e-6;
        if (ks > 1) t += (double)M * N * 4.0 * (ks + 1) / hbm + 3e-6;
        return t * 1e6;
    };
    GemmCand all[4 * 4];
    int n = 0;   // at most 4 tiles x 4 K splits
    double pen0 = 1.0;
    const int t0 = pick_tile(M, N, f32), k0 = gemm_ksplit(M, N, K, c_dt);
    for (int i = 0; i < nt; ++i) {
        if (ts[i].id == t0) pen0 = ts[i].pen;
        for (int ks = 1; ks <= 8; ks *= 2) {
            if (!plan_candidate(M, N, K, ts[i].id, ks, c_dt)) continue;
            all[n++] = GemmCand{ts[i].id, ks, cost(ts[i].id, ks, ts[i].pen)};
        }
    }
    // the analytic pick first, then the rest by modelled time
    const GemmCand head{t0, k0, cost(t0, k0, pen0)};
    int w = 0;
    GemmCand rest[4 * 4];
    for (int i = 0; i < n; ++i)
        if (!(all[i].tile == t0 && all[i].ksplit == k0)) rest[w++] = all[i];
    std::sort(rest, rest + w, [](const GemmCand& a, const GemmCand& b) { return a.cost < b.cost; });
    int m = 0;
    out[m++] = head;
    for (int i = 0; i < w && m < max_out && m < 7; ++i) out[m++] = rest[i];
    return m;
}

// ---- few token rows: one workgroup per 16 output features ----------------------
// y[0:M, n0:n0+16] = round_out(post * (scale * (af . bf^T) + a . b^T) + b) for
// M <= 32 with fp32 accumulation and all of K in one workgroup, so that no
// K split and no second kernel are needed.  Wave w of the NW takes the w-th
// share of the 64-byte K steps, reading its fragments of W (a) and x (b)
// straight from global memory D steps ahead: every fragment is used by one
// wave once, so nothing is staged in LDS.  Wave 0 also takes the fold, first,
// as the tiled kernel does.  The waves' sums meet in LDS in wave order.
// (x is read by every workgroup: beyond 32 rows that L2 traffic outgrows W's
// and the tiled kernel with its K split is faster.)
template <class CT, int MT, int D, int NW>
__global__ __launch_bounds__(64 * NW) void skinny_kernel(GemmParams p) {
    __shared__ __attribute__((aligned(16))) f32x4 red[NW - 1][MT][64];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t n0 = (int64_t)blockIdx.x * 16;
    const uint32_t kb = (uint32_t)(p.K * CT::es);   // bytes of a row
    const int nrows = (int)(p.N - n0 < 16 ? p.N - n0 : 16);
    const auto rw = make_rsrc_uniform((const char*)p.a + n0 * kb, (uint32_t)nrows * kb);
    const auto rx = make_rsrc_uniform(p.b, (uint32_t)(p.M * kb));
    const uint32_t lo = (uint32_t)(lane >> 4) * 16;        // the lane's 16 bytes of a 64-byte step
    const uint32_t wrow = (uint32_t)(lane & 15) * kb + lo;
    f32x4 acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (wave == 0 && p.rf > 0) {
        // fold: scale * (up rows n0.. . h rows^T), rank padded with zeros
        const uint32_t fb = (uint32_t)(p.rf * CT::es);
        const auto ru = make_rsrc_uniform((const char*)p.af + n0 * fb, (uint32_t)nrows * fb);
        const auto rh = make_rsrc_uniform(p.bf, (uint32_t)(p.M * fb));
        for (uint32_t f = 0; f < fb; f += 64) {
            const i32x4 ua = buf_load16(ru, f + lo < fb ? (uint32_t)(lane & 15) * fb + f + lo : OOB);
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                const i32x4 hb = buf_load16(rh, f + lo < fb ? (uint32_t)(16 * t + (lane & 15)) * fb + f + lo : OOB);
                acc[t] = CT::step(ua, hb, acc[t]);
            }
        }
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[t] *= p.scale;
    }

    // the wave's K steps, D in flight: ring slot u holds step s0 + u (mod D);
    // the run is padded to a multiple of D with steps that read zeros, so the
    // loop body has no exit in it (the compiler then keeps the ring in flight
    // across iterations instead of waiting for all of it at the loop head)
    const int steps = (int)((kb + 63) / 64);
    const int s0 = steps * wave / NW, s1 = steps * (wave + 1) / NW;
    const int se = s0 + ((s1 - s0 + D - 1) / D) * D;
    i32x4 wa[D], xa[D][MT];
#pragma unroll
    for (int u = 0; u < D; ++u) {
        const uint32_t k = (uint32_t)(s0 + u) * 64;
        const bool in = s0 + u < s1 && k + lo < kb;
        wa[u] = buf_load16(rw, in ? wrow + k : OOB);
#pragma unroll
        for (int t = 0; t < MT; ++t) xa[u][t] = buf_load16(rx, in ? (uint32_t)(16 * t + (lane & 15)) * kb + lo + k : OOB);
    }
    for (int sb = s0; sb < se; sb += D) {
#pragma unroll
        for (int u = 0; u < D; ++u) {
#pragma unroll
            for (int t = 0; t < MT; ++t) acc[t] = CT::step(wa[u], xa[u][t], acc[t]);
            const int sn = sb + u + D;
            const uint32_t k = (uint32_t)sn * 64;
            const bool in = sn < s1 && k + lo < kb;
            wa[u] = buf_load16(rw, in ? wrow + k : OOB);
#pragma unroll
            for (int t = 0; t < MT; ++t) xa[u][t] = buf_load16(rx, in ? (uint32_t)(16 * t + (lane & 15)) * kb + lo + k : OOB);
        }
    }

    if (wave > 0) {
#pragma unroll
        for (int t = 0; t < MT; ++t) red[wave - 1][t][lane] = acc[t];
    }
    __syncthreads();
    if (wave != 0) return;
    // lane: rows m = 16 t + (lane & 15), features n0 + 4 (lane >> 4) .. +3
    const int64_t nb = n0 + 4 * (lane >> 4);
    float bias[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) bias[e] = (p.bias != nullptr && nb + e < p.N) ? load_as_f32(p.bias, p.bias_dt, nb + e) : 0.f;
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        f32x4 sum = acc[t];
#pragma unroll
        for (int w = 0; w < NW - 1; ++w) sum += red[w][t][lane];
        const int64_t m = 16 * t + (lane & 15);
        if (m >= p.M) continue;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = sum[e] * p.post + bias[e];
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
            const uint32_t l2 = p.y_dt == DT_F16 ? pack_f16x2(v[0], v[1]) : pack_bf16x2(v[0], v[1]);
            const uint32_t h2 = p.y_dt == DT_F16 ? pack_f16x2(v[2], v[3]) : pack_bf16x2(v[2], v[3]);
            uint16_t* y = (uint16_t*)p.y;
            if (p.vec_store && nb + 3 < p.N) {
                *(i32x2*)(y + base) = i32x2{(int)l2, (int)h2};
            } else {
                const uint16_t o[4] = {(uint16_t)l2, (uint16_t)(l2 >> 16), (uint16_t)h2, (uint16_t)(h2 >> 16)};
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (nb + e < p.N) y[base + e] = o[e];
            }
        }
    }
}

template <class CT>
static hipError_t run_skinny(const GemmParams& p, hipStream_t s) {
    const int64_t kb = p.K * CT::es, fb = p.rf * CT::es;
    if (kb % 16 != 0 || fb % 16 != 0 || p.M * kb >= ((int64_t)1 << 31) || 16 * kb >= ((int64_t)1 << 31) ||
        p.M * fb >= ((int64_t)1 << 31) || 16 * fb >= ((int64_t)1 << 31))
        return hipErrorInvalidValue;
    const dim3 g((unsigned)((p.N + 15) / 16));
    // (4 waves: 8, each with the same ring, measured slower at 16 x 3072 x 3072)
    if (p.M <= 16) hipLaunchKernelGGL((skinny_kernel<CT, 1, 8, 4>), g, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((skinny_kernel<CT, 2, 6, 4>), g, dim3(256), 0, s, p);
    return hipGetLastError();
}

// the few-row kernel takes the forward's plain case: no gain, operands as
// rows, 16-byte row pieces, 32-bit offsets
bool gemm_skinny(int c_dt, const GemmParams& p) {
    if (p.M < 1 || p.M > 32 || p.gain != nullptr || p.ta || p.tb || p.tile != GEMM_TILE_AUTO) return false;
    const int64_t es = c_dt == DT_F32 ? 4 : 2, kb = p.K * es, fb = p.rf * es;
    return kb % 16 == 0 && fb % 16 == 0 && p.M * kb < ((int64_t)1 << 31) && 16 * kb < ((int64_t)1 << 31) &&
           p.M * fb < ((int64_t)1 << 31) && 16 * fb < ((int64_t)1 << 31);
}

hipError_t launch_gemm(int c_dt, const GemmParams& p, hipStream_t s) {
    if (p.skinny && gemm_skinny(c_dt, p)) {
        if (c_dt == DT_F16) return run_skinny<CF16>(p, s);
        if (c_dt == DT_BF16) return run_skinny<CBF16>(p, s);
        return run_skinny<CF32>(p, s);
    }
    int t = p.tile >= 0 ? p.tile : pick_tile(p.M, p.N, c_dt == DT_F32);
    if (c_dt == DT_F32 && t != T_M && t != T_S) return hipErrorInvalidValue;   // no fp32 instance
    if (p.ta || p.tb) {
        // transposed operands: both of them, 16-bit compute, no fold, no 192-row tile
        if (c_dt == DT_F32 || !p.ta || !p.tb || p.rf > 0) return hipErrorInvalidValue;
        if (t == T_G) t = T_L;
    }
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
