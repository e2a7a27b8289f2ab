// hpass.hip -- contractions whose result is rounded to a 16-bit format and
// then used again, so that the rounding decision must be the one the exact
// value gets:
//   * h = x_c . down_c^T, rounded to the compute (storage) dtype before its
//     second dot (LyCORIS "Precision" page, "Measured accuracy");
//   * the plain affine projection p = x_c . W_c^T, rounded to the output dtype
//     before the bias is added (Luminal FP16 page, "What Was Fixed").
// A value that lands on the wrong side of a rounding midpoint moves by one
// 16-bit ulp, and the following sum (bias, or the whole bypass row) can cancel
// down to where that ulp is far outside any per-element tolerance.
//
// Method (16-bit compute).  K is cut into blocks of 64.  In each block a row
// of x and a row of b (down_c or W_c) are split as v = v_hi + v_lo, v_hi the
// value rounded to the grid 2^(e-8), e = floor(log2 max|v|) over the block
// (v_hi is at most 2^9 grid units and representable in either 16-bit format).
//   hh:    b_hi . x_hi   every product is an integer times the block's grid
//                        product with magnitude <= 2^18, so every partial sum
//                        of the block's 64 products is an integer of magnitude
//                        at most 2^24 times that grid: exact in fp32 however
//                        the MFMA orders or aligns its additions.  Added to an
//                        fp64 accumulator once per block (exact).
//   cross: b_lo . x + b_hi . x_lo   small (|v_lo| <= 2^(e-9)); one MFMA chain
//                        per 32-k step, the block's two chains added in fp32
//                        and then to the fp64 accumulator.
// Both sums of a column block are added to the fp64 accumulator while the
// MFMAs of the next column block run (the conversions and fp64 adds are a
// large part of the vector work, and they then overlap the matrix pipe).
// gfx950 MFMA steps keep about two bits below the ulp of their running sum
// and truncate (measured), so a step adding terms of total magnitude S to an
// accumulator C errs by less than 18 * 2^-24 * (|C| + S); the cross chain of
// a 32-k step therefore errs by less than 36 * 2^-24 * S_chain, the fp32 sum
// of a block's two chains adds at most 2^-24 * (S_0 + S_1) (1 + 36 * 2^-24),
// and over all blocks (Cauchy-Schwarz on the sums of |products|)
//   E(m, j) = 38 * 2^-24 * (|x_m| |b_lo,j| + |x_lo,m| (|b_j| + |b_lo,j|)) + fp64 slack
//             + K * 2^-120 (fp32 underflow: products of bf16 values far below 1),
// with |x_m| and |x_lo,m| the diagonals of the MFMA Gram matrices of x and
// x_lo (inflated by their own step error) and the norms of b from the
// preparation pass.
// When [h - E, h + E] straddles a rounding boundary of the 16-bit format, the
// element goes on the workgroup's work list in LDS; after the outputs are
// stored, the workgroup's waves take the list in groups and overwrite each
// listed output with the value rounded from the fp64 dot product of its x row
// and b row (products exact, batched 16-byte loads).  fp32 compute, or an
// fp32 rounding target, needs no guard: a flip there moves the result by
// 2^-24 relative.
//
// Work split: a workgroup owns RW*16 rows and RP = 16*JB*CG columns; its
// waves form RW row groups x KS k groups x CG column groups (k group g takes
// the blocks g, g+KS, ...; partial sums meet in LDS at the end).  The b_hi,
// b_lo and x tiles of KS blocks at a time are staged through LDS straight
// from global memory, several rounds ahead.
#include "kernels.h"
#include "lyc_device.h"

#ifndef LYC_R16_KS
#define LYC_R16_KS 8
#endif

namespace lyc {

// Error of one MFMA step, in units of 2^-24 of |accumulator| + sum|products|
// (measured bound), and of a block's cross sum, in units of 2^-24 of its
// absolute sums: two chains of two steps (2 * STEP_ERR) and the fp32 add of
// the two (1, rounded up to leave room for the second-order term).
constexpr double STEP_ERR = 18.0;
constexpr double GUARD_CROSS = 2.0 * STEP_ERR + 2.0;

// The guard's per-column factors: with n = |x_m| and n_lo = |x_lo,m| (each
// inflated by `slack`), the bound is E = n P + n_lo Q + D, where
//   P = slack |scale| (GUARD_CROSS 2^-24 |b_lo,j| + 2^-37 |b_j|),
//   Q = slack |scale| GUARD_CROSS 2^-24 (|b_j| + |b_lo,j|),
// D the underflow term.  |b_lo,j| = inf (a block of b that could not be
// split) makes P infinite, which flags the column.
__device__ __forceinline__ double2 guard_pq(double b, double bl, double as) {
    const double slack = 1.0 + 0x1p-20;
    return double2{slack * as * (0x1p-24 * GUARD_CROSS * bl + 0x1p-37 * b), slack * as * 0x1p-24 * GUARD_CROSS * (b + bl)};
}

template <class CT>
__device__ __forceinline__ float unpack_lo(uint32_t u) {
    return CT::dt == DT_F16 ? f16_to_f32((uint16_t)u) : bf16_to_f32((uint16_t)u);
}
template <class CT>
__device__ __forceinline__ float unpack_hi(uint32_t u) {
    return CT::dt == DT_F16 ? f16_to_f32((uint16_t)(u >> 16)) : __builtin_bit_cast(float, u & 0xffff0000u);
}
// two floats that are exactly representable in the 16-bit format -> packed pair
template <class CT>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    if (CT::dt == DT_F16) return (uint32_t)f32_to_f16(a) | ((uint32_t)f32_to_f16(b) << 16);
    return (__builtin_bit_cast(uint32_t, a) >> 16) | (__builtin_bit_cast(uint32_t, b) & 0xffff0000u);
}

// largest |value| among the 8 16-bit values of a fragment, as its bit pattern
// (for finite values the magnitude order is the integer order without the sign)
__device__ __forceinline__ uint32_t absmax_bits(i32x4 v) {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t u = (uint32_t)v[i] & 0x7fff7fffu;
        const uint32_t lo = u & 0xffffu, hi = u >> 16;
        m = m > lo ? m : lo;
        m = m > hi ? m : hi;
    }
    return m;
}

// maximum of v over the lanes l, l^16, l^32 and l^48 (the four lanes that
// hold one row of a 64-k block in the MFMA fragment layout), with gfx950's row
// swaps: v_permlane16_swap of v with itself hands lane l of rows 0 and 1 (2
// and 3) the values of rows 0 and 1 (2 and 3) at its position, and
// v_permlane32_swap does the same for the two halves.  Plain vector
// instructions: a shuffle through the LDS crossbar (ds_bpermute) took a round
// trip each, twice at the start of every k block.
__device__ __forceinline__ uint32_t max_row_lanes(uint32_t v) {
    const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    const uint32_t m = a[0] > a[1] ? a[0] : a[1];
    const auto b = __builtin_amdgcn_permlane32_swap(m, m, false, false);
    return b[0] > b[1] ? b[0] : b[1];
}

// grid exponent g = floor(log2 m) - 8 of a positive 16-bit magnitude m (bits)
template <class CT>
__device__ __forceinline__ int grid_exp(uint32_t m) {
    if (CT::dt == DT_F16) {
        const int E = (int)(m >> 10);
        const int e = E > 0 ? E - 15 : (31 - __builtin_clz(m | 1u)) - 24;
        return e - 8;
    }
    const int E = (int)(m >> 7);
    const int e = E > 0 ? E - 127 : (31 - __builtin_clz(m | 1u)) - 133;
    return e - 8;
}

// Split a fragment on the grid 2^g (round to nearest): hi on the grid, lo = v - hi.
// Adding and subtracting magic = 1.5 * 2^(g+23) rounds an fp32 value of
// magnitude below 2^(g+22) to a multiple of 2^g.
template <class CT>
__device__ __forceinline__ void split16(i32x4 v, float magic, i32x4& hi, i32x4& lo) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t u = (uint32_t)v[i];
        const float a = unpack_lo<CT>(u), b = unpack_hi<CT>(u);
        const float ah = (a + magic) - magic, bh = (b + magic) - magic;
        hi[i] = (int)pack2<CT>(ah, bh);
        lo[i] = (int)pack2<CT>(a - ah, b - bh);
    }
}

// The same split for fp16 in packed fp16 arithmetic (three v_pk_add_f16 per
// 4 bytes instead of the unpack / fp32 / repack sequence): with
// M = 1.5 * 2^(g+10), v + M lies in (1, 2) * 2^(g+10) for |v| < 2^(g+9) and
// rounds to a multiple of 2^g (ties to even; 2^(g+11) at most), t - M is
// exact, and so is v - hi (2^g is a multiple of the ulp of every v of the
// block, and hi = 0 wherever |v| < 2^(g-1)).
// The sum stays finite and M is a normal fp16 value for g <= 4 (callers
// check: at g = 5 values just below 2^14 would round v + M up to 2^16, which
// overflows fp16), and a grid finer
// than fp16's smallest subnormal 2^-24 is taken as 2^-24 (every value of such
// a block is on it: hi = v, lo = 0).
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
__device__ __forceinline__ void split16_pk(i32x4 v, int g, i32x4& hi, i32x4& lo) {
    const int gc = g < -24 ? -24 : g;
    const _Float16 M = __builtin_bit_cast(_Float16, (uint16_t)(((gc + 25) << 10) | 0x200));
    const f16x8_t vv = __builtin_bit_cast(f16x8_t, v);
    const f16x8_t h = (vv + M) - M;
    hi = __builtin_bit_cast(i32x4, h);
    lo = __builtin_bit_cast(i32x4, vv - h);
}

// exact products of two 16-byte fragments, summed in fp64 (two chains)
template <class CT>
__device__ __forceinline__ double dot16_f64(i32x4 a, i32x4 b) {
    double s0 = 0.0, s1 = 0.0;
    if (CT::dt == DT_F32) {
        const f32x4 fa = __builtin_bit_cast(f32x4, a), fb = __builtin_bit_cast(f32x4, b);
        s0 = __builtin_fma((double)fa[0], (double)fb[0], s0);
        s1 = __builtin_fma((double)fa[1], (double)fb[1], s1);
        s0 = __builtin_fma((double)fa[2], (double)fb[2], s0);
        s1 = __builtin_fma((double)fa[3], (double)fb[3], s1);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t ua = (uint32_t)a[i], ub = (uint32_t)b[i];
            s0 = __builtin_fma((double)unpack_lo<CT>(ua), (double)unpack_lo<CT>(ub), s0);
            s1 = __builtin_fma((double)unpack_hi<CT>(ua), (double)unpack_hi<CT>(ub), s1);
        }
    }
    return s0 + s1;
}

template <class CT>
__device__ __forceinline__ uint16_t round16(double v) {
    return CT::dt == DT_F16 ? f64_to_f16(v) : f64_to_bf16(v);
}

// the projection rounded to the output dtype (exactly, from the fp64 value), as fp32
template <class CT>
__device__ __forceinline__ float affine_value(double acc, int out_dt) {
    if (out_dt == DT_F32) return (float)acc;   // one rounding, fp64 -> fp32
    if (CT::dt == DT_F16) return f16_to_f32(round16<CT>(acc));
    return bf16_to_f32(round16<CT>(acc));
}

// fp64 dot products of K-contiguous row pairs (exact products), 64 / L pairs
// per wave: lane j of an L-lane group takes the 16-byte chunks j, j + L, ...
// of its group's pair; the loads of up to B chunks per row per lane are issued
// together, so that each batch costs one memory round trip.  Every lane of a
// group gets its group's sum.  L is a power of two, uniform over the wave.
template <class CT, int B>
__device__ __forceinline__ double group_dot(const i32x4* xrow, const i32x4* brow, uint32_t nch, int j, int L) {
    double s0 = 0.0, s1 = 0.0;
    for (uint32_t c0 = (uint32_t)j; c0 < nch; c0 += (uint32_t)(L * B)) {
        i32x4 xv[B], bv[B];
#pragma unroll
        for (int i = 0; i < B; ++i) {
            const uint32_t c = c0 + (uint32_t)(L * i);
            xv[i] = c < nch ? xrow[c] : i32x4{0, 0, 0, 0};
            bv[i] = c < nch ? brow[c] : i32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < B; i += 2) {
            s0 += dot16_f64<CT>(xv[i], bv[i]);
            s1 += dot16_f64<CT>(xv[i + 1], bv[i + 1]);
        }
    }
    double part = s0 + s1;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        if (o < L) part += __shfl_xor(part, o);
    return part;
}

// element e (lane-dependent) of a 4-vector, by bit masks: a conditional chain
// here becomes branches.  The whole vector is bit_cast (a bit_cast of one
// element of a vector is folded to element 0 by this compiler).
__device__ __forceinline__ float pick4(f32x4 v, int e) {
    const i32x4 u = __builtin_bit_cast(i32x4, v);
    uint32_t r = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) r |= (uint32_t)u[i] & (0u - (uint32_t)(e == i));
    return __builtin_bit_cast(float, r);
}

// Epilogue of one wave's accumulators, for the column blocks in `owned` (a
// wave-uniform bit mask; the k groups split a workgroup's blocks): rounding
// guard (flagged elements are appended to the workgroup's work list), then
// h_r or the affine output.
template <class CT, int JB, bool SB>
__device__ __forceinline__ void xr_epilogue(const XrParams& p, double (&acc)[JB][4], double xm2, double xl2, bool wide,
                                            int64_t wg_m0, int64_t j0, int my_row, int c0, int cols_wg, int lane,
                                            unsigned* lcount, uint32_t* list, const float (&bsq)[SB ? JB : 1][2],
                                            const double2* lbn, const float* lbias, uint32_t owned) {
    constexpr bool SPLIT = CT::dt != DT_F32;
    const int64_t m = wg_m0 + my_row;
    const bool row_ok = m < p.M;
    // the bias (plain affine form), from the workgroup's copy in LDS (zero
    // past the last column).  The affine form runs with JB = 4; wider
    // instances never read it.
    float bias[JB][4] = {};
    if (JB <= 4 && p.mode != XR_H && p.bias != nullptr) {
#pragma unroll
        for (int i = 0; i < JB * 4; ++i) bias[i >> 2][i & 3] = lbias[c0 + (i >> 2) * 16 + 4 * (lane >> 4) + (i & 3)];
    }

    // guard: flag the elements whose error interval straddles a rounding
    // boundary (bit jb*4+e of `flags`); they are re-evaluated after the
    // outputs are written, so the accumulators are only ever indexed statically.
    // r16 = round16(h - E) is the rounded value wherever the element is not
    // flagged (rounding is monotone: round(h - E) <= round(h) <= round(h + E)).
    uint32_t flags = 0;
    uint16_t r16[JB][4];
    if (SPLIT) {
        const bool guard = p.guard != 0;
        const double slack = 1.0 + 0x1p-20;
        const double xn2 = __builtin_sqrt(xm2) * slack;
        const double xln = __builtin_sqrt(xl2) * slack;
        // h = scale * C: the bound scales with |scale| (the fp64 product's own
        // rounding, 2^-53 relative, lies far inside the 2^-37 slack term)
        const double as = __builtin_fabs(p.scale);
        // fp32 products and partial sums below 2^-126 (bf16 operands far
        // below 1) may be flushed, or rounded on fp32's subnormal grid, and a
        // grid product below 2^-149 makes the hi.hi sums inexact: either way
        // an MFMA step loses less than 33 * 2^-126 (32 products and its
        // result), and an element takes 6 steps per 64-k block, so an
        // absolute K * 2^-120 covers the whole contraction
        const double D = (double)p.K * 0x1p-120 * as;
#pragma unroll
        for (int jb = 0; jb < JB; ++jb) {
            if (!((owned >> jb) & 1u)) continue;   // (uniform: another k group's block)
            double2 pq[4];   // the guard's factors {P, Q} of the lane's 4 columns of this block
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int jl = c0 + jb * 16 + 4 * (lane >> 4) + e;
                if constexpr (SB) {
                    // the lane's column c of this block: its row's squared norms
                    // sit in lane c (shuffled whatever the lane's own columns)
                    const int c = 4 * (lane >> 4) + e;
                    const float vb = __shfl(bsq[SB ? jb : 0][0], c), vl = __shfl(bsq[SB ? jb : 0][1], c);
                    const double2 v = guard_pq(__builtin_sqrt((double)vb) * slack,
                                               vl < __builtin_inff() ? __builtin_sqrt((double)vl) * slack
                                                                     : __builtin_inf(),
                                               as);
                    pq[e] = (guard && jl < cols_wg) ? v : double2{0.0, 0.0};
                } else {
                    pq[e] = (guard && jl < cols_wg) ? lbn[jl] : double2{0.0, 0.0};
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int jl = c0 + jb * 16 + 4 * (lane >> 4) + e;
                const double h = acc[jb][e] * p.scale;
                const double E = __builtin_fma(xn2, pq[e].x, __builtin_fma(xln, pq[e].y, D));
                const uint16_t lo = round16<CT>(h - E);
                r16[jb][e] = lo;
                // (the second conversion stays conditional: computed for every
                // element up front, the 8-block instance runs out of registers)
                const bool bwide = !(pq[e].x < 1e300);   // a block of b could not be split
                const bool flag = (guard & row_ok & (jl < cols_wg)) && (wide || bwide || lo != round16<CT>(h + E));
                flags |= (uint32_t)flag << (jb * 4 + e);
            }
        }
        // guarded elements go to the workgroup's work list: one LDS atomic per lane
        if (flags != 0u) {
            unsigned at = atomicAdd(lcount, (unsigned)__builtin_popcount(flags));
            for (uint32_t f = flags; f != 0u; f &= f - 1u) {
                const int bit = __builtin_ctz(f);
                list[at++] = ((uint32_t)my_row << 16) | (uint32_t)(c0 + (bit >> 2) * 16 + 4 * (lane >> 4) + (bit & 3));
            }
        }
    }

    if (row_ok) {
        if (p.mode == XR_H) {
            // h_r [M][ld_out] in the compute dtype (all RP columns, padding included)
#pragma unroll
            for (int jb = 0; jb < JB; ++jb) {
                if (!((owned >> jb) & 1u)) continue;
                const int64_t jg = j0 + c0 + jb * 16 + 4 * (lane >> 4);
                if (CT::dt == DT_F32) {
                    float* hp = (float*)p.out + m * p.ld_out + jg;
                    *(f32x4*)hp = f32x4{(float)(acc[jb][0] * p.scale), (float)(acc[jb][1] * p.scale),
                                        (float)(acc[jb][2] * p.scale), (float)(acc[jb][3] * p.scale)};
                } else {
                    uint16_t* hp = (uint16_t*)p.out + m * p.ld_out + jg;
                    *(i32x2*)hp = i32x2{(int)(r16[jb][0] | ((uint32_t)r16[jb][1] << 16)),
                                        (int)(r16[jb][2] | ((uint32_t)r16[jb][3] << 16))};
                }
            }
        } else {
            // plain affine: y = round_out(round_out(p) + b); the projection
            // rounds to fp32 for an fp32 output, else to the compute dtype (= output)
#pragma unroll
            for (int jb = 0; jb < JB; ++jb) {
                if (!((owned >> jb) & 1u)) continue;
                const int jl0 = c0 + jb * 16 + 4 * (lane >> 4);
                const int64_t n0 = j0 + jl0;
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float pr;
                    if (!SPLIT || p.out_dt == DT_F32) pr = (float)acc[jb][e];
                    else pr = CT::dt == DT_F16 ? f16_to_f32(r16[jb][e]) : bf16_to_f32(r16[jb][e]);
                    v[e] = pr + bias[jb][e];
                }
                const int64_t base = m * p.ld_out + n0;
                if (p.out_dt == DT_F32) {
                    float* y = (float*)p.out;
                    if (p.vec_store && jl0 + 3 < cols_wg) {
                        *(f32x4*)(y + base) = f32x4{v[0], v[1], v[2], v[3]};
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (jl0 + e < cols_wg) y[base + e] = v[e];
                    }
                } else {
                    const uint32_t lo = p.out_dt == DT_F16 ? pack_f16x2(v[0], v[1]) : pack_bf16x2(v[0], v[1]);
                    const uint32_t hi = p.out_dt == DT_F16 ? pack_f16x2(v[2], v[3]) : pack_bf16x2(v[2], v[3]);
                    uint16_t* y = (uint16_t*)p.out;
                    if (p.vec_store && jl0 + 3 < cols_wg) {
                        *(i32x2*)(y + base) = i32x2{(int)lo, (int)hi};
                    } else {
                        const uint16_t o[4] = {(uint16_t)lo, (uint16_t)(lo >> 16), (uint16_t)hi, (uint16_t)(hi >> 16)};
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (jl0 + e < cols_wg) y[base + e] = o[e];
                    }
                }
            }
        }
    }
}

// LDS pipeline of the contraction: a round stages KS k blocks of 128 bytes,
// each with its b tile(s) (RP rows; b_hi and b_lo under the split) and its x
// tile (RW*16 rows), all filled straight from global memory.  The workgroup's
// NW = 4*CG waves are RW row groups x KS k groups x CG column groups; a wave
// owns 16 rows and JB*16 columns.
// row groups of a workgroup with KS k groups: 4 / KS (16 rows per group), at least 1
constexpr int xr_row_groups(int KS) { return KS >= 4 ? 1 : 4 / KS; }

template <int JB, int KS, int CG, int RW_, bool SPLIT, bool SB = false>
struct XrStage {
    static constexpr int NB = (SPLIT && !SB) ? 2 : 1;   // b_hi and b_lo tiles, or b itself
    static constexpr int RW = RW_, RP = JB * 16 * CG, NW = RW * KS * CG;
    static constexpr int TILE = RP * 128, XT = RW * 16 * 128;
    static constexpr int BYTES = KS * (NB * TILE + XT);
    static constexpr int NBB = KS * NB * RP / 8;      // 1 KiB wave loads of b per round
    static constexpr int NBLK = NBB + KS * RW * 2;    // ... of b and x
    static constexpr int Q = NBLK / NW;               // per wave
    static constexpr int NS = 4 * BYTES <= 159 * 1024 ? 4 : (3 * BYTES <= 159 * 1024 ? 3 : 2);
    static_assert(NBLK % NW == 0, "loader split");
    static_assert(NS * BYTES <= 160 * 1024 && (NS - 1) * Q < 64, "LDS stages");
};

// SB (plain affine form, and h at rank 16 with down in the compute dtype):
// b = W_c or down_c is loaded as stored and split in the kernel
// exactly as x is (per 64-k block of each row), its row norms taken from the
// diagonals of MFMA Gram matrices; no preparation pass.  The guard's count is
// then written per workgroup (p.flagged[workgroup], a plain store), so that
// nothing needs clearing beforehand.
template <class CT, int JB, int KS, int CG, int RW_, bool SB = false>
__global__ __launch_bounds__(64 * RW_ * KS * CG) __attribute__((amdgpu_num_vgpr(256)))
void xr_kernel(XrParams p) {
    constexpr bool SPLIT = CT::dt != DT_F32;     // 16-bit compute: hi/lo split and guard
    static_assert(!SB || (SPLIT && JB <= 4), "in-kernel split of b: 16-bit compute, at most 4 column blocks");
    using ST = XrStage<JB, KS, CG, RW_, SPLIT, SB>;
    constexpr int NB = ST::NB, RW = ST::RW, RP = ST::RP, TILE = ST::TILE, NS = ST::NS, Q = ST::Q, NW = ST::NW;
    __shared__ __attribute__((aligned(16))) char sd[NS * ST::BYTES];
    const int tid = threadIdx.x, lane = tid & 63;
    // wave index in a scalar register: everything derived from it stays uniform
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rg = wave % RW, kg = (wave / RW) % KS, cg = wave / (RW * KS);
    const int c0 = cg * JB * 16;                // the wave's first column within the workgroup
    const int64_t wg_m0 = (int64_t)blockIdx.x * (RW * 16);
    const int64_t j0 = (int64_t)blockIdx.y * RP;
    const int rows_wg = (int)((p.M - wg_m0) < RW * 16 ? (p.M - wg_m0) : RW * 16);
    const int cols_wg = (int)((p.Nc - j0) < RP ? (p.Nc - j0) : RP);
    const uint32_t kbytes = (uint32_t)(p.K * CT::es);
    const int my_row = rg * 16 + (lane & 15);   // row within the workgroup
    const auto rsx = make_rsrc((const char*)p.x + wg_m0 * kbytes, (uint32_t)rows_wg * kbytes);
    const auto rsh = make_rsrc((const char*)p.b + j0 * kbytes, (uint32_t)cols_wg * kbytes);
    const auto rsl = make_rsrc((const char*)((SPLIT && !SB) ? p.b_lo : p.b) + j0 * kbytes, (uint32_t)cols_wg * kbytes);

    double acc[JB][4];
#pragma unroll
    for (int jb = 0; jb < JB; ++jb)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[jb][e] = 0.0;
    double xm2 = 0.0, xl2 = 0.0;   // |x_m|^2 and |x_lo,m|^2 of this lane's row (16-bit compute)
    f32x4 gx = f32x4{0.f, 0.f, 0.f, 0.f}, gl = f32x4{0.f, 0.f, 0.f, 0.f};   // Gram accumulators
    // SB: Gram accumulators of the b rows of each column block (b and b_lo), and
    // whether a block of the lane's b row could not be split
    constexpr int JBS = SB ? JB : 1;
    f32x4 gbb[JBS], gbl[JBS];
    bool wideb[JBS];
#pragma unroll
    for (int jb = 0; jb < JBS; ++jb) {
        gbb[jb] = f32x4{0.f, 0.f, 0.f, 0.f};
        gbl[jb] = f32x4{0.f, 0.f, 0.f, 0.f};
        wideb[jb] = false;
    }

    const int KT = (int)((kbytes + 127) / 128);   // k blocks of 128 bytes
    const int ROUNDS = (KT + KS - 1) / KS;
    // Wave load blk of a round fills 1 KiB = 8 rows x 128 bytes of LDS: blocks
    // below NBB belong to b tile t = blk / (RP/8) (k group t / NB, array t % NB),
    // the rest to the x tile of k group (blk - NBB) / (2 RW).  Lane l fetches the
    // chunk that the swizzled layout (lds_off) puts in its slot.
    const uint32_t kc16 = (uint32_t)((lane & 7) ^ (lane >> 3)) << 4;
    uint32_t voff[Q];   // offset of the lane's chunk within its array, k block 0
    uint32_t kpos[Q];   // byte position of that chunk within a row, k block 0
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const int blk = wave + q * NW;
        int g, row;
        if (blk < ST::NBB) {
            const int t = blk / (RP / 8);
            g = t / NB;
            row = (blk % (RP / 8)) * 8 + (lane >> 3);
        } else {
            const int xb = blk - ST::NBB;
            g = xb / (RW * 2);
            row = (xb % (RW * 2)) * 8 + (lane >> 3);
        }
        kpos[q] = (uint32_t)g * 128 + kc16;
        voff[q] = (uint32_t)row * kbytes + kpos[q];
    }
    auto stage_at = [&](int r) { return sd + (r % NS) * ST::BYTES; };
#define LYC_ISSUE_LOADS(ST_, KB0_, V_)                                                              \
    _Pragma("unroll") for (int q = 0; q < Q; ++q) {                                                 \
        const int blk = wave + q * NW;                                                              \
        const uint32_t v = V_;                                                                      \
        auto* dst = (__attribute__((address_space(3))) void*)((ST_) + blk * 1024);                  \
        if (blk >= ST::NBB) __builtin_amdgcn_raw_ptr_buffer_load_lds(rsx, dst, 16, v, (int)(KB0_), 0, 0); \
        else if ((blk / (RP / 8)) % NB) __builtin_amdgcn_raw_ptr_buffer_load_lds(rsl, dst, 16, v, (int)(KB0_), 0, 0); \
        else __builtin_amdgcn_raw_ptr_buffer_load_lds(rsh, dst, 16, v, (int)(KB0_), 0, 0);          \
    }
    // (a round that lies wholly inside K takes no per-lane range test)
#define LYC_ISSUE_ROUND(R)                                                                          \
    do {                                                                                            \
        char* st_ = stage_at(R);                                                                    \
        const uint32_t kb0_ = (uint32_t)((R) * KS) * 128;                                           \
        if (kb0_ + KS * 128 <= kbytes) {                                                            \
            LYC_ISSUE_LOADS(st_, kb0_, voff[q])                                                     \
        } else {                                                                                    \
            LYC_ISSUE_LOADS(st_, kb0_, kb0_ + kpos[q] < kbytes ? voff[q] : OOB)                     \
        }                                                                                           \
    } while (0)

    bool wide = false;   // a block beyond the split's exponent range: re-evaluate the row
    // hi.hi sum and the two cross sums of the column block before the current
    // one (16-bit compute, b split beforehand; after a k block's last column
    // block, those of JB - 1), added to acc while the current one's MFMAs run
    f32x4 phh = f32x4{0.f, 0.f, 0.f, 0.f}, pc0 = phh, pc1 = phh;
    if (ROUNDS > 0) {
        // rounds 0 .. NS-1 fill every stage; round 0 must land
#pragma unroll
        for (int r0 = 0; r0 < NS; ++r0)
            if (r0 < ROUNDS) LYC_ISSUE_ROUND(r0);
        if (NS - 1 < ROUNDS) wait_vm<(NS - 1) * Q>();
        else wait_vm<0>();
        lds_barrier();
    }
    for (int r = 0; r < ROUNDS; ++r) {
        const char* cur = stage_at(r);
        const char* th = cur + (kg * NB) * TILE;                       // this k group's b_hi (or b) tile
        const char* xs = cur + KS * NB * TILE + kg * (RW * 16 * 128);  // this k group's x tile
        i32x4 xr[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) xr[s] = *(const i32x4*)(xs + lds_off(my_row, s * 4 + (lane >> 4)));
        // (b split beforehand) the first column block's b fragments {hi, lo} x
        // {k half 0, 1}, read with x's so that their latency overlaps the split
        i32x4 bq[4];
        const int kc0 = lane >> 4, rl = c0 + (lane & 15);
        if constexpr (SPLIT && !SB) {
            const char* tl0 = th + TILE;
            bq[0] = *(const i32x4*)(th + lds_off(rl, kc0));
            bq[1] = *(const i32x4*)(tl0 + lds_off(rl, kc0));
            bq[2] = *(const i32x4*)(th + lds_off(rl, 4 + kc0));
            bq[3] = *(const i32x4*)(tl0 + lds_off(rl, 4 + kc0));
            __builtin_amdgcn_sched_barrier(0);   // (issued here, not after the split)
        }
        if (SPLIT) {
            // block maximum of |x| for the lane's row (4 lane groups x 16 values)
            uint32_t mb = absmax_bits(xr[0]);
            const uint32_t m1 = absmax_bits(xr[1]);
            mb = mb > m1 ? mb : m1;
            mb = max_row_lanes(mb);
            const int g = grid_exp<CT>(mb);
            wide |= (g > 100);
            i32x4 xh[2], xlo[2];
            if (CT::dt == DT_F16 && __all(g <= 4)) {
                split16_pk(xr[0], g, xh[0], xlo[0]);
                split16_pk(xr[1], g, xh[1], xlo[1]);
            } else {
                const float magic = __builtin_ldexpf(1.5f, (g > 100 ? 100 : g) + 23);
                split16<CT>(xr[0], magic, xh[0], xlo[0]);
                split16<CT>(xr[1], magic, xh[1], xlo[1]);
            }
            // squared norms of the wave's rows of x and x_lo: the diagonals of
            // their 16 x 16 Gram matrices, accumulated by the MFMA
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                gx = CT::step(xr[s], xr[s], gx);
                gl = CT::step(xlo[s], xlo[s], gl);
            }
            const char* tl = th + TILE;             // this k group's b_lo tile
            if constexpr (SB) {
#pragma unroll
                for (int jb = 0; jb < JB; ++jb) {
                    const int row = c0 + jb * 16 + (lane & 15);
                    i32x4 br[2], bsh[2], bsl[2];   // this block's b row and its split
#pragma unroll
                    for (int s = 0; s < 2; ++s) br[s] = *(const i32x4*)(th + lds_off(row, s * 4 + (lane >> 4)));
                    uint32_t mbb = absmax_bits(br[0]);
                    const uint32_t n1 = absmax_bits(br[1]);
                    mbb = mbb > n1 ? mbb : n1;
                    mbb = max_row_lanes(mbb);
                    const int gb = grid_exp<CT>(mbb);
                    wideb[SB ? jb : 0] |= (gb > 100);
                    if (CT::dt == DT_F16 && __all(gb <= 4)) {
                        split16_pk(br[0], gb, bsh[0], bsl[0]);
                        split16_pk(br[1], gb, bsh[1], bsl[1]);
                    } else {
                        const float magic = __builtin_ldexpf(1.5f, (gb > 100 ? 100 : gb) + 23);
                        split16<CT>(br[0], magic, bsh[0], bsl[0]);
                        split16<CT>(br[1], magic, bsh[1], bsl[1]);
                    }
                    f32x4 hh = f32x4{0.f, 0.f, 0.f, 0.f}, cs = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < 2; ++s) {
                        gbb[SB ? jb : 0] = CT::step(br[s], br[s], gbb[SB ? jb : 0]);
                        gbl[SB ? jb : 0] = CT::step(bsl[s], bsl[s], gbl[SB ? jb : 0]);
                        hh = CT::step(bsh[s], xh[s], hh);                                   // exact
                        f32x4 cx = CT::step(bsl[s], xr[s], f32x4{0.f, 0.f, 0.f, 0.f});      // cross chain
                        cx = CT::step(bsh[s], xlo[s], cx);
#pragma unroll
                        for (int e = 0; e < 4; ++e) cs[e] = s == 0 ? cx[e] : cs[e] + cx[e];
                    }
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        acc[jb][e] += (double)hh[e];
                        acc[jb][e] += (double)cs[e];
                    }
                }
            } else {
                // b fragments of a column block, read one column block ahead
                // (the first with x's); each column block's MFMAs share their
                // stretch of the schedule with the fold of the previous one's sums
#pragma unroll
                for (int jb = 0; jb < JB; ++jb) {
                    // the previous column block's sums enter this stretch here (an
                    // empty asm pins them, so the fold below cannot move up to
                    // the MFMAs that produce them)
                    asm volatile("" : "+v"(phh), "+v"(pc0), "+v"(pc1));
                    i32x4 bn[4];
                    if (jb + 1 < JB) {
                        const int rn = rl + (jb + 1) * 16;
                        bn[0] = *(const i32x4*)(th + lds_off(rn, kc0));
                        bn[1] = *(const i32x4*)(tl + lds_off(rn, kc0));
                        bn[2] = *(const i32x4*)(th + lds_off(rn, 4 + kc0));
                        bn[3] = *(const i32x4*)(tl + lds_off(rn, 4 + kc0));
                    }
                    const f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
                    f32x4 hh = CT::step(bq[0], xh[0], z);          // exact
                    f32x4 c0 = CT::step(bq[1], xr[0], z);          // cross chains
                    f32x4 c1 = CT::step(bq[3], xr[1], z);
                    hh = CT::step(bq[2], xh[1], hh);
                    c0 = CT::step(bq[0], xlo[0], c0);
                    c1 = CT::step(bq[2], xlo[1], c1);
                    const int pj = jb == 0 ? JB - 1 : jb - 1;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        acc[pj][e] += (double)phh[e];
                        acc[pj][e] += (double)(pc0[e] + pc1[e]);
                    }
                    // ... and the fold is done before the stretch ends
                    asm volatile("" : "+v"(acc[pj][0]), "+v"(acc[pj][1]), "+v"(acc[pj][2]), "+v"(acc[pj][3]));
                    phh = hh;
                    pc0 = c0;
                    pc1 = c1;
                    if (jb + 1 < JB) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) bq[i] = bn[i];
                    }
                    // MFMA, then a few vector ops, in turn (next fragments' reads first)
                    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
                    for (int i = 0; i < 6; ++i) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        } else {
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int kc = s * 4 + (lane >> 4);
#pragma unroll
                for (int jb = 0; jb < JB; ++jb) {
                    const i32x4 bf = *(const i32x4*)(th + lds_off(c0 + jb * 16 + (lane & 15), kc));
                    const f32x4 c = CT::step(bf, xr[s], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[jb][e] += (double)c[e];
                }
            }
        }
        if (r + 1 < ROUNDS) {
            // round r+1 must land (NS-2 rounds after it may be in flight); then
            // refill the stage just read with round r+NS
            if (r + NS - 1 < ROUNDS) wait_vm<(NS - 2) * Q>();
            else wait_vm<0>();
            lds_barrier();
            if (r + NS < ROUNDS) LYC_ISSUE_ROUND(r + NS);
        }
    }
#undef LYC_ISSUE_ROUND
#undef LYC_ISSUE_LOADS
    if (SPLIT && !SB) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc[JB - 1][e] += (double)phh[e];
            acc[JB - 1][e] += (double)(pc0[e] + pc1[e]);
        }
    }
    // The epilogue's per-column inputs, one per thread: the guard's factors
    // from the norms {|b|, |b_lo|} (b split beforehand) and the bias (plain
    // affine form).
    // Their loads are issued here and land in LDS with the k groups' partial
    // sums, so that one memory round trip overlaps the reduction (read in the
    // epilogue, each lane's 4 JB columns would take JB round trips in turn).
    static_assert(64 * NW >= RP, "one thread per column");
    const bool ld_bn = SPLIT && !SB && p.guard && tid < cols_wg;
    const bool ld_bias = p.mode != XR_H && p.bias != nullptr && tid < RP;
    double2 bnv = double2{0.0, 0.0};
    float biasv = 0.f;
    if (ld_bn) bnv = p.bnorm[j0 + tid];
    if (ld_bias && tid < cols_wg) biasv = load_as_f32(p.bias, p.bias_dt, j0 + tid);
    __syncthreads();   // every wave is done with the stages (they hold the k-group reduction next)

    // LDS after the main loop: [k-group reduction][count][work list of guarded
    // elements][column guard factors][bias].  The k groups' partial sums meet
    // column block by column block: block jb belongs to k group jb % KS, and
    // every wave writes the partial sums of the blocks it does not own (SLOTS
    // of them) and the statistics of its rows (NST values), so that the
    // epilogue's work is spread over all k groups.
    constexpr int SLOTS = JB - JB / KS;
    constexpr int NST = 3 + (SB ? JB * 2 : 0);
    constexpr int W = SLOTS * 4 + NST;
    constexpr int RED = KS > 1 ? KS * CG * RW * 64 * W * 8 : 0;
    constexpr int CAP = RW * 16 * RP;                      // every element of the workgroup
    static_assert(RED + 16 + CAP * 4 + RP * 20 <= NS * ST::BYTES, "reduction buffer, work list, column inputs");
    unsigned* lcount = (unsigned*)(sd + RED);
    uint32_t* list = (uint32_t*)(sd + RED + 16);
    double2* lbn = (double2*)(sd + RED + 16 + CAP * 4);
    float* lbias = (float*)(sd + RED + 16 + CAP * 4 + RP * 16);
    if (tid == 0) *lcount = 0u;
    if (ld_bn) lbn[tid] = guard_pq(bnv.x, bnv.y, __builtin_fabs(p.scale));
    if (ld_bias) lbias[tid] = biasv;

    if (SPLIT) {
        // Gram diagonal: row r of the wave sits in lane r + 16 (r >> 2), element
        // r & 3.  The MFMA steps' error (below STEP * 2^-24 of |accumulator| +
        // sum|products| per step, every term >= 0, so at most (steps + 1) STEP
        // 2^-24 relative) is covered by inflating, and products that underflowed
        // by 2^-120 per step (a step adds 32 squares per element).
        const int r = lane & 15, e = r & 3;
        const float dx = pick4(gx, e), dl = pick4(gl, e);
        const int src = r + 16 * (r >> 2);
        const double steps = 2.0 * ROUNDS;
        const double infl = 1.0 + 2.0 * STEP_ERR * 0x1p-24 * (steps + 1.0) + 0x1p-20;
        xm2 = (double)__shfl(dx, src) * infl + steps * 0x1p-120;
        xl2 = (double)__shfl(dl, src) * infl + steps * 0x1p-120;
    }
    // SB: the same for the b rows of every column block (lane l: the row
    // l & 15 of the block; |b_lo|^2 = inf where a block of the row could not
    // be split); the epilogue takes its columns' values from those lanes
    float bsq[JBS][2];
    if constexpr (SB) {
        const int r = lane & 15, e = r & 3;
        const int src = r + 16 * (r >> 2);
        const double steps = 2.0 * ROUNDS;
        const double infl = 1.0 + 2.0 * STEP_ERR * 0x1p-24 * (steps + 1.0) + 0x1p-20;
#pragma unroll
        for (int jb = 0; jb < JB; ++jb) {
            const float db = __shfl(pick4(gbb[jb], e), src), dlo = __shfl(pick4(gbl[jb], e), src);
            bsq[jb][0] = (float)((double)db * infl + steps * 0x1p-120);
            bsq[jb][1] = wideb[jb] ? __builtin_inff() : (float)((double)dlo * infl + steps * 0x1p-120);
        }
    }
    // meet the k groups' partial sums in LDS (the B tiles are no longer needed):
    // slot t of wave g holds the t-th block among those g does not own
    uint32_t owned = 0;
#pragma unroll
    for (int jb = 0; jb < JB; ++jb) owned |= (uint32_t)(jb % KS == kg) << jb;
    if (KS > 1) {
        double* red = (double*)sd;                 // [KS][CG][RW][64 lanes][W]
        double* dst = red + ((size_t)((kg * CG + cg) * RW + rg) * 64 + lane) * W;
        int t = 0;
#pragma unroll
        for (int jb = 0; jb < JB; ++jb) {
            if ((owned >> jb) & 1u) continue;
#pragma unroll
            for (int e = 0; e < 4; ++e) dst[t * 4 + e] = acc[jb][e];
            ++t;
        }
        double* st = dst + SLOTS * 4;
        st[0] = xm2;
        st[1] = xl2;
        st[2] = wide ? 1.0 : 0.0;
        if constexpr (SB) {
#pragma unroll
            for (int jb = 0; jb < JB; ++jb) {
                st[3 + 2 * jb] = bsq[jb][0];
                st[3 + 2 * jb + 1] = bsq[jb][1];
            }
        }
    }
    __syncthreads();   // partial sums, the cleared count and the column inputs are visible
    if (KS > 1 && owned != 0u) {   // (a wave without blocks, where KS > JB, has nothing to sum)
        // each owned block and the row statistics summed over the k groups in
        // the order 0, 1, ..., KS-1 (the wave's own part from its registers)
        const double* red = (const double*)sd;
#pragma unroll
        for (int jb = 0; jb < JB; ++jb) {
            if (!((owned >> jb) & 1u)) continue;   // (uniform)
            double t4[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
            for (int g2 = 0; g2 < KS; ++g2) {
                // block jb's slot in wave g2 (which does not own it): jb less
                // the blocks below jb that g2 owns
                const int t = jb - (jb > g2 ? (jb - 1 - g2) / KS + 1 : 0);
                const double* src = red + ((size_t)((g2 * CG + cg) * RW + rg) * 64 + lane) * W + t * 4;
#pragma unroll
                for (int e = 0; e < 4; ++e) t4[e] += g2 == kg ? acc[jb][e] : src[e];
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[jb][e] = t4[e];
        }
        double txm = 0.0, txl = 0.0;
        bool twide = false;
        float tb[JBS][2];
#pragma unroll
        for (int jb = 0; jb < JBS; ++jb) tb[jb][0] = tb[jb][1] = 0.f;
#pragma unroll
        for (int g2 = 0; g2 < KS; ++g2) {
            const bool mine = g2 == kg;
            const double* st = red + ((size_t)((g2 * CG + cg) * RW + rg) * 64 + lane) * W + SLOTS * 4;
            txm += mine ? xm2 : st[0];
            txl += mine ? xl2 : st[1];
            twide |= mine ? wide : st[2] != 0.0;
            if constexpr (SB) {
                // (the fp32 sums are rounded up by the epilogue's slack)
#pragma unroll
                for (int jb = 0; jb < JB; ++jb) {
                    tb[jb][0] = (float)((double)tb[jb][0] + (mine ? bsq[jb][0] : (float)st[3 + 2 * jb]));
                    tb[jb][1] = (float)((double)tb[jb][1] + (mine ? bsq[jb][1] : (float)st[3 + 2 * jb + 1]));
                }
            }
        }
        xm2 = txm;
        xl2 = txl;
        wide = twide;
        if constexpr (SB) {
#pragma unroll
            for (int jb = 0; jb < JB; ++jb) {
                bsq[jb][0] = tb[jb][0];
                bsq[jb][1] = tb[jb][1];
            }
        }
    }
    if (owned != 0u)
        xr_epilogue<CT, JB, SB>(p, acc, xm2, xl2, wide, wg_m0, j0, my_row, c0, cols_wg, lane, lcount, list, bsq, lbn,
                                lbias, owned);
    // The guarded elements: every wave takes its share of the list and
    // overwrites the stored output with the value rounded from the fp64 dot
    // product.  The barrier's release makes the first stores complete before.
    __syncthreads();
    if (SPLIT && p.guard) {
        const unsigned n = *lcount;
        const uint32_t nch = kbytes / 16;
        const i32x4* xbase = (const i32x4*)((const char*)p.x + wg_m0 * kbytes);
        const i32x4* bbase = (const i32x4*)((const char*)p.b_full + j0 * kbytes);
        // entries per wave and pass: as many (up to 8) as keep every lane's
        // share of a row within one batch of B chunks (one memory round trip
        // per pass; the accumulators are dead by now)
        constexpr int B = 16;
        const int G = nch <= 8 * B ? 8 : (nch <= 16 * B ? 4 : (nch <= 32 * B ? 2 : 1));
        const int L = 64 / G, j = lane & (L - 1);
        for (unsigned i0 = (unsigned)(wave * G); i0 < n; i0 += (unsigned)(ST::NW * G)) {
            const unsigned i = i0 + (unsigned)(lane / L);
            const bool mine = i < n;
            const uint32_t ent = list[mine ? i : i0];
            const int row = (int)(ent >> 16), col = (int)(ent & 0xffffu);
            const double d = group_dot<CT, B>(xbase + (size_t)row * nch, bbase + (size_t)col * nch, nch, j, L);
            if (mine && j == 0) {
                const int64_t m = wg_m0 + row, j = j0 + col;
                if (p.mode == XR_H) {
                    ((uint16_t*)p.out)[m * p.ld_out + j] = round16<CT>(d * p.scale);
                } else {
                    const float bias = p.bias != nullptr ? load_as_f32(p.bias, p.bias_dt, j) : 0.f;
                    const float v = affine_value<CT>(d, p.out_dt) + bias;
                    // the guard runs for 16-bit outputs only
                    ((uint16_t*)p.out)[m * p.ld_out + j] = p.out_dt == DT_F16 ? f32_to_f16(v) : f32_to_bf16(v);
                }
            }
        }
        if (SB || p.flag_per_wg) {
            if (tid == 0) p.flagged[blockIdx.y * gridDim.x + blockIdx.x] = n;
        } else {
            if (tid == 0 && n) atomicAdd(p.flagged, n);
        }
    } else if ((SB || p.flag_per_wg) && tid == 0) {
        p.flagged[blockIdx.y * gridDim.x + blockIdx.x] = 0u;   // no guard: nothing re-evaluated
    }
}

template <class CT, int JB, int KS, int CG, int RW = xr_row_groups(KS), bool SB = false>
static hipError_t run_xr(const XrParams& p, hipStream_t s) {
    constexpr int RP = JB * 16 * CG;
    const dim3 grid((unsigned)((p.M + RW * 16 - 1) / (RW * 16)), (unsigned)((p.Nc + RP - 1) / RP));
    // per-workgroup guard counts: the caller's slots must cover the grid
    if ((SB || p.flag_per_wg) && (int64_t)grid.x * grid.y > p.flag_slots) return hipErrorInvalidValue;
    hipLaunchKernelGGL((xr_kernel<CT, JB, KS, CG, RW, SB>), grid, dim3(64 * RW * KS * CG), 0, s, p);
    return hipGetLastError();
}

// k groups: the fewest that still give one workgroup per CU (256), at most 4
static int pick_ks(int64_t M, int64_t col_tiles) {
    int ks = 1;
    while (ks < 4 && ((M + 64 / ks - 1) / (64 / ks)) * col_tiles < 256) ks *= 2;
    return ks;
}

// KSMAX 8: where 16 rows per workgroup are needed, 8 k groups (two waves per
// SIMD) instead of 4
template <class CT, int JB, int CG, int KSMAX, bool SB = false>
static hipError_t run_xr_jb(const XrParams& p, hipStream_t s) {
    const int64_t col_tiles = (p.Nc + JB * 16 * CG - 1) / (JB * 16 * CG);
    const int ks = pick_ks(p.M, col_tiles);
    constexpr int K2 = KSMAX >= 2 ? 2 : 1, K4 = KSMAX >= 4 ? KSMAX : 1;
    // (with b split in the kernel, one b tile per stage: a single k group's
    // loads would not divide among its waves, so it takes two)
    if constexpr (!SB) {
        if (ks == 1 || KSMAX == 1) return run_xr<CT, JB, 1, CG, xr_row_groups(1), SB>(p, s);
    }
    if (ks <= 2 || KSMAX == 2) return run_xr<CT, JB, K2, CG, xr_row_groups(K2), SB>(p, s);
    return run_xr<CT, JB, K4, CG, xr_row_groups(K4), SB>(p, s);
}

// The plain affine form under 16-bit compute: 64 x 64 tiles (8 waves, two k
// groups) where there are at least 256 of them, W split beforehand by the
// row-norm pass (its four row-group waves would each split the same 64 W rows
// again: measured 28.5 + 7.1 us against 40.6 us in one launch at
// 1024 x 768 x 1024); else 16-column workgroups with up to 8 k groups and W
// split in the kernel (one launch: 19.0 -> 12.0 us at M = 16, 24.4 -> 15.7 us
// at M = 128).  Returns the latter launch's workgroup count (its guard-count
// slots), or 0 where the row-norm pass is used.
static int64_t xr_split_b_wgs(int64_t M, int64_t Nc) {
    const int64_t col_tiles = (Nc + 15) / 16;
    const int ks = pick_ks(M, col_tiles);
    const int rw = ks <= 2 ? xr_row_groups(2) : xr_row_groups(8);   // run_xr_jb<CT, 1, 1, 8, true>
    return ((M + rw * 16 - 1) / (rw * 16)) * col_tiles;
}

int64_t xr_affine_workgroups(int64_t M, int64_t N) {
    const int64_t t64 = ((M + 63) / 64) * ((N + 63) / 64);
    if (t64 >= 256) return 0;
    return xr_split_b_wgs(M, N);
}

// the 64 x 64 tiles of run_xr<CT, 4, 2, 1, 4> (W split beforehand)
int64_t xr_affine_split_pass_workgroups(int64_t M, int64_t N) { return ((M + 63) / 64) * ((N + 63) / 64); }

// h at rank 16 with down already in the compute dtype: the same 16-column
// launch with down split in the kernel, so that no preparation pass runs
int64_t xr_h_split_b_workgroups(int64_t M, int64_t Nc) { return Nc == 16 ? xr_split_b_wgs(M, Nc) : 0; }

// Columns per wave (JB blocks of 16), column groups (CG), k groups (KS) and
// row groups (RW) per workgroup: at least 256 workgroups where M allows,
// eight waves (two per SIMD) for the wider ranks, and one wave over all
// columns of its rows where that fits, so that each x fragment is split once.
template <class CT>
static hipError_t run_xr_ct(const XrParams& p, hipStream_t s) {
    if (p.mode == XR_AFFINE) {
        // 16-bit compute: the launches xr_affine_workgroups describes; fp32
        // compute keeps the 4-wave 64-column split
        if constexpr (CT::dt != DT_F32) {
            if (((p.M + 63) / 64) * ((p.Nc + 63) / 64) >= 256) return run_xr<CT, 4, 2, 1, 4>(p, s);
            return run_xr_jb<CT, 1, 1, 8, true>(p, s);
        }
        return run_xr_jb<CT, 4, 1, 4>(p, s);
    }
    if (p.split_b) {
        if constexpr (CT::dt != DT_F32) {
            if (p.Nc == 16) return run_xr_jb<CT, 1, 1, 8, true>(p, s);
        }
        return hipErrorInvalidValue;
    }
    switch (p.Nc) {
    case 16:   // 16-bit compute only (fp32 compute pads the rank to 32)
        if (CT::dt == DT_F32) return hipErrorInvalidValue;
        return run_xr_jb<CT, (CT::dt == DT_F32 ? 2 : 1), 1, LYC_R16_KS>(p, s);
    case 32: return run_xr_jb<CT, 2, 1, 4>(p, s);
    case 64:
        // one wave per 16 rows x all 64 columns where M fills the GPU with
        // 32- or 64-row workgroups (the x split is done once per row)
        if (p.M >= 256 * 64) return run_xr<CT, 4, 2, 1, 4>(p, s);
        if (p.M >= 256 * 32) return run_xr<CT, 4, 4, 1, 2>(p, s);
        return run_xr_jb<CT, 2, 2, 4>(p, s);
    case 128:
        if (p.M >= 256 * 64) return run_xr<CT, 8, 2, 1, 4>(p, s);
        return run_xr_jb<CT, 4, 2, 2>(p, s);
    case 256: return run_xr<CT, 8, 1, 2>(p, s);
    default: return hipErrorInvalidValue;
    }
}

// ---- few token rows: one wave per h element ------------------------------------
// With few rows of x the split contraction above is latency-bound: one
// workgroup walks all of K.  There each element h[m][j] gets a wave of its
// own instead: the fp64 dot of x_m and down_j (exact products; lane l takes
// the 16-byte chunks l, l + 64, ..., then a butterfly over the lanes), with a
// bound on that sum's own rounding error, gamma_n * sum|p| (n: the longest
// chain of additions a product goes through).  Where [s - E, s + E] straddles
// a rounding boundary of the compute dtype, the wave sums again carrying each
// addition's rounding error (TwoSum) and rounds that compensated sum, whose
// error is of the order of 2^-100 sum|p|.  Workgroup w writes the number of
// such elements to slot w of p.flagged (no clearing needed).
template <class CT>
__device__ __forceinline__ void vals_f64(i32x4 v, double (&o)[CT::dt == DT_F32 ? 4 : 8]) {
    if constexpr (CT::dt == DT_F32) {
        const f32x4 f = __builtin_bit_cast(f32x4, v);
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = (double)f[i];
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            o[2 * i] = (double)unpack_lo<CT>((uint32_t)v[i]);
            o[2 * i + 1] = (double)unpack_hi<CT>((uint32_t)v[i]);
        }
    }
}

__device__ __forceinline__ double load_widen(const void* base, int dt, int64_t i) {
    if (dt == DT_F32) return (double)((const float*)base)[i];
    const uint16_t b = ((const uint16_t*)base)[i];
    return (double)(dt == DT_F16 ? f16_to_f32(b) : bf16_to_f32(b));
}

// s + t = a + b exactly (Knuth's TwoSum)
__device__ __forceinline__ void two_sum(double a, double b, double& s, double& t) {
    s = a + b;
    const double bb = s - a;
    t = (a - (s - bb)) + (b - bb);
}

template <class CT>
__global__ __launch_bounds__(256) void hdot_kernel(HdotParams p) {
    constexpr int V = CT::dt == DT_F32 ? 4 : 8;   // values per 16-byte chunk
    const int lane = threadIdx.x & 63;
    const int64_t e = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);   // element m * r_pad + j
    __shared__ unsigned wflag[4];
    unsigned straddled = 0;
    if (e < p.M * p.r_pad) {
        const int64_t m = e / p.r_pad;
        const int j = (int)(e % p.r_pad);
        double v = 0.0;
        if (j < p.rank) {
            const char* xr = (const char*)p.x + m * p.K * CT::es;
            const char* dr = (const char*)p.down + (int64_t)j * p.K * CT::es;
            // lane sums: s (the dot) and a (sum of |products|), and the chain length n
            double s = 0.0, a = 0.0;
            int64_t n;
            if (p.vec) {
                // 4 chunks of each row per lane in flight at a time: one memory
                // round trip per 4 (the chunk order of the sums is unchanged)
                const int64_t nch = p.K / V;
                for (int64_t c0 = lane; c0 < nch; c0 += 4 * 64) {
                    i32x4 xq[4], dq[4];
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        const int64_t c = c0 + 64 * b;
                        xq[b] = c < nch ? ((const i32x4*)xr)[c] : i32x4{0, 0, 0, 0};
                        dq[b] = c < nch ? ((const i32x4*)dr)[c] : i32x4{0, 0, 0, 0};
                    }
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        double xv[V], dv[V];
                        vals_f64<CT>(xq[b], xv);
                        vals_f64<CT>(dq[b], dv);
#pragma unroll
                        for (int i = 0; i < V; ++i) {
                            s = __builtin_fma(xv[i], dv[i], s);
                            a = __builtin_fma(__builtin_fabs(xv[i]), __builtin_fabs(dv[i]), a);
                        }
                    }
                }
                n = ((nch + 63) / 64) * V;
            } else {
                for (int64_t k = lane; k < p.K; k += 64) {
                    const double xv = load_widen(p.x, CT::dt, m * p.K + k), dv = load_widen(p.down, CT::dt, (int64_t)j * p.K + k);
                    s = __builtin_fma(xv, dv, s);
                    a = __builtin_fma(__builtin_fabs(xv), __builtin_fabs(dv), a);
                }
                n = (p.K + 63) / 64;
            }
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) {
                s += __shfl_xor(s, o, 64);
                a += __shfl_xor(a, o, 64);
            }
            s = __shfl(s, 0, 64);   // every lane takes lane 0's sums (the butterfly's orders differ)
            a = __shfl(a, 0, 64);
            n += 6;
            const double u = 0x1p-53, g = (double)n * u / (1.0 - (double)n * u);
            const double E = g * a * (1.0 + 2.0 * g) + 0x1p-1060;
            bool cross;
            if constexpr (CT::dt == DT_F32) cross = (float)(s - E) != (float)(s + E);
            else cross = round16<CT>(s - E) != round16<CT>(s + E);
            v = s;
            if (cross) {
                straddled = 1;
                double S = 0.0, C = 0.0, t, err;
                if (p.vec) {
                    const int64_t nch = p.K / V;
                    for (int64_t c = lane; c < nch; c += 64) {
                        double xv[V], dv[V];
                        vals_f64<CT>(((const i32x4*)xr)[c], xv);
                        vals_f64<CT>(((const i32x4*)dr)[c], dv);
#pragma unroll
                        for (int i = 0; i < V; ++i) {
                            two_sum(S, xv[i] * dv[i], t, err);   // the product is exact
                            S = t;
                            C += err;
                        }
                    }
                } else {
                    for (int64_t k = lane; k < p.K; k += 64) {
                        two_sum(S, load_widen(p.x, CT::dt, m * p.K + k) * load_widen(p.down, CT::dt, (int64_t)j * p.K + k),
                                t, err);
                        S = t;
                        C += err;
                    }
                }
#pragma unroll
                for (int o = 32; o >= 1; o >>= 1) {
                    const double So = __shfl_xor(S, o, 64), Co = __shfl_xor(C, o, 64);
                    two_sum(S, So, t, err);
                    S = t;
                    C = (C + Co) + err;
                }
                v = __shfl(S, 0, 64) + __shfl(C, 0, 64);
            }
        }
        if (lane == 0) {
            const int64_t at = m * p.r_pad + j;
            if constexpr (CT::dt == DT_F32) ((float*)p.out)[at] = (float)v;
            else ((uint16_t*)p.out)[at] = round16<CT>(v);
        }
    }
    if (lane == 0) wflag[threadIdx.x >> 6] = straddled;
    __syncthreads();
    if (threadIdx.x == 0) p.flagged[blockIdx.x] = wflag[0] + wflag[1] + wflag[2] + wflag[3];
}

int64_t hdot_workgroups(int64_t M, int64_t r_pad) { return (M * r_pad + 3) / 4; }

hipError_t launch_hdot(int c_dt, const HdotParams& p, hipStream_t s) {
    const int64_t g = hdot_workgroups(p.M, p.r_pad);
    if (g <= 0) return hipSuccess;
    if (g > 65535) return hipErrorInvalidValue;
    if (c_dt == DT_F16) hipLaunchKernelGGL(hdot_kernel<CF16>, dim3((unsigned)g), dim3(256), 0, s, p);
    else if (c_dt == DT_BF16) hipLaunchKernelGGL(hdot_kernel<CBF16>, dim3((unsigned)g), dim3(256), 0, s, p);
    else hipLaunchKernelGGL(hdot_kernel<CF32>, dim3((unsigned)g), dim3(256), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_xr(int c_dt, const XrParams& p, hipStream_t s) {
    if (c_dt == DT_F16) return run_xr_ct<CF16>(p, s);
    if (c_dt == DT_BF16) return run_xr_ct<CBF16>(p, s);
    return run_xr_ct<CF32>(p, s);
}

}  // namespace lyc
