// lyc_device.h -- device-side building blocks shared by the gfx950 kernels:
// vector types, IEEE round-to-nearest-even conversions, buffer resources and
// the MFMA step for each compute dtype.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lyc {

enum : int { DT_F16 = 1, DT_BF16 = 2, DT_F32 = 3 };

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

// ---- scalar conversions ------------------------------------------------------

__device__ __forceinline__ float f16_to_f32(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __builtin_bit_cast(float, (uint32_t)b << 16); }

// fp32 -> fp16, round to nearest even (v_cvt_f16_f32 under the default mode;
// subnormal results kept, overflow to inf).
__device__ __forceinline__ uint16_t f32_to_f16(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 under the default
// mode, subnormals kept; identical to rounding the bit pattern for all 2^32
// inputs, NaN to a NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// Two fp32 values -> a packed pair of 16-bit values (a in the low half), round
// to nearest even: one v_cvt_pk_{f16,bf16}_f32.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, f16x2_t));
}
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

__device__ __forceinline__ float load_as_f32(const void* p, int dt, int64_t i) {
    if (dt == DT_F32) return ((const float*)p)[i];
    uint16_t b = ((const uint16_t*)p)[i];
    return dt == DT_F16 ? f16_to_f32(b) : bf16_to_f32(b);
}

// N elements idx[i] of a vector of n >= 1 elements stored in dtype dt,
// widened to fp32 (0 where idx[i] >= n).  All N loads are issued, unmasked at
// clamped indices, before the first conversion: around a per-element dtype
// switch the compiler waits for each load before issuing the next.
template <int N>
__device__ __forceinline__ void load_n_as_f32(const void* p, int dt, const int64_t (&idx)[N], int64_t n,
                                              float (&out)[N]) {
    uint32_t raw[N];
    if (dt == DT_F32) {
#pragma unroll
        for (int i = 0; i < N; ++i) raw[i] = ((const uint32_t*)p)[idx[i] < n ? idx[i] : n - 1];
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i) raw[i] = ((const uint16_t*)p)[idx[i] < n ? idx[i] : n - 1];
    }
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const float v = dt == DT_F32 ? __builtin_bit_cast(float, raw[i])
                                     : (dt == DT_F16 ? f16_to_f32((uint16_t)raw[i]) : bf16_to_f32((uint16_t)raw[i]));
        out[i] = idx[i] < n ? v : 0.f;
    }
}

// binary64 -> binary32 rounded to odd: the value truncated toward zero, with
// the last significand bit set when that truncation was inexact.  Rounding
// this to nearest even in a format with at least two fewer significand bits
// gives the same result as rounding the binary64 value directly (Boldo and
// Melquiond, "Emulation of FMA and correctly rounded sums: proved algorithms
// using rounding to odd", IEEE Trans. Computers 2008).  Valid where the
// binary32 result is normal, |d| >= 2^-126 (the conversion may flush
// subnormal results).  Overflow gives the largest finite binary32 value
// (odd), which then overflows either 16-bit format.  Branch-free.
__device__ __forceinline__ float f64_to_f32_odd(double d) {
    const float f = (float)d;   // round to nearest even
    const double back = (double)f;
    const uint32_t u = __builtin_bit_cast(uint32_t, f);
    const uint32_t t = u - (__builtin_fabs(back) > __builtin_fabs(d) ? 1u : 0u);   // toward zero
    return (back == d || d != d) ? f : __builtin_bit_cast(float, t | 1u);
}

// binary64 -> fp16 / bf16, round to nearest even, one rounding from the
// binary64 value; subnormal results kept, overflow to inf, NaN stays NaN.
// Below 2^-126: fp16 gives a signed zero (its smallest subnormal is 2^-24);
// bf16 rounds on its subnormal grid 2^-133 by adding and subtracting
// 1.5 * 2^-81, whose binary64 ulp is that grid.
__device__ __forceinline__ uint16_t f64_to_f16(double d) {
    const uint16_t r = f32_to_f16(f64_to_f32_odd(d));
    const uint16_t z = (uint16_t)((__builtin_bit_cast(uint64_t, d) >> 48) & 0x8000u);
    return __builtin_fabs(d) < 0x1p-126 ? z : r;
}
__device__ __forceinline__ uint16_t f64_to_bf16(double d) {
    const uint16_t r = f32_to_bf16(f64_to_f32_odd(d));
    const double q = (d + 0x1.8p-81) - 0x1.8p-81;   // a multiple of 2^-133, |q| <= 2^-126
    const uint16_t t = (uint16_t)((uint32_t)(__builtin_fabs(q) * 0x1p133) |
                                  (uint32_t)((__builtin_bit_cast(uint64_t, d) >> 48) & 0x8000u));
    return __builtin_fabs(d) < 0x1p-126 ? t : r;
}

// ---- buffer resources (hardware range checking: out-of-range loads read 0) --

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// A buffer resource from values the compiler may hold in vector registers:
// each piece is taken from the first lane (they are uniform), so that the
// loads through it need no per-lane loop.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc_uniform(const void* base, uint32_t bytes) {
    const uint64_t b = (uint64_t)base;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
    return make_rsrc((const void*)(((uint64_t)hi << 32) | lo), __builtin_amdgcn_readfirstlane(bytes));
}

// ---- tiles stored with the contraction index as rows (transposing LDS reads) --

// Chunk permutation of a transposed tile's row r (CPR 16-byte chunks a row):
// 32-byte pairs of chunks move by a row-dependent amount so that the rows one
// half-wave's transposing read touches (r = 0..3 and 8..11 of a group of 16,
// or 4..7 and 12..15) fall on distinct banks.  Rows of 256 bytes or more
// start on the same bank, so the pair index takes bits 0, 1 and 3 of r; rows
// of 128 bytes alternate halves of the banks, so it takes bits 1 and 3.
template <int CPR>
__device__ __forceinline__ int tswz(int r) {
    static_assert(CPR >= 8, "transposed tile rows of 128 bytes or more");
    if constexpr (CPR >= 16) return 2 * ((r & 3) | ((r >> 1) & 4));
    else return 2 * (((r >> 1) & 1) | ((r >> 2) & 2));
}

// 8 consecutive contraction indices of one column from a transposed tile:
// two transposing reads.  Lane l (group G = l/16, j = l%16) addresses row
// 8G + j/4 (+4) and column base + 4 (j%4); the read hands lane l the values of
// column base + l%16 for rows 8G .. 8G+3 (+4), the MFMA operand layout.
template <int ROWS>
__device__ __forceinline__ i32x4 frag_t(const char* tile, int row0, int col0, int lane) {
    typedef short s4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s4 lds_s4;
    const int G = lane >> 4, j = lane & 15;
    const int col = col0 + 4 * (j & 3);
    const int r1 = row0 + 8 * G + (j >> 2), r2 = r1 + 4;
    const char* p1 = tile + r1 * (ROWS * 2) + (((col >> 3) ^ tswz<ROWS / 8>(r1)) << 4) + ((col >> 2) & 1) * 8;
    const char* p2 = tile + r2 * (ROWS * 2) + (((col >> 3) ^ tswz<ROWS / 8>(r2)) << 4) + ((col >> 2) & 1) * 8;
    const s4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(__attribute__((address_space(3))) char*)p1);
    const s4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(__attribute__((address_space(3))) char*)p2);
    const i32x2 ai = __builtin_bit_cast(i32x2, a), bi = __builtin_bit_cast(i32x2, b);
    return i32x4{ai[0], ai[1], bi[0], bi[1]};
}

// An offset that is always beyond num_records (which stays below 2^31).
constexpr uint32_t OOB = 0x80000000u;

__device__ __forceinline__ i32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

// ---- MFMA per compute dtype ---------------------------------------------------
// One "step" consumes, per lane, one 16-byte fragment of A and of B:
//  16-bit: v_mfma_f32_16x16x32_{f16,bf16}: the 8 elements are 8 k values.
//  fp32:   four v_mfma_f32_16x16x4_f32, element e of each lane's 4 floats in
//          the e-th instruction (A and B take the same element, so every
//          (n,m) pair meets each k exactly once).
// Output layout (16x16 blocks): lane l, register e holds row 4*(l>>4)+e of the
// A side and column l&15 of the B side.

struct CF16 {
    static constexpr int dt = DT_F16;
    static constexpr int es = 2;
    __device__ static __forceinline__ f32x4 step(i32x4 a, i32x4 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                      0, 0, 0);
    }
};
struct CBF16 {
    static constexpr int dt = DT_BF16;
    static constexpr int es = 2;
    __device__ static __forceinline__ f32x4 step(i32x4 a, i32x4 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                       c, 0, 0, 0);
    }
};
struct CF32 {
    static constexpr int dt = DT_F32;
    static constexpr int es = 4;
    __device__ static __forceinline__ f32x4 step(i32x4 a, i32x4 b, f32x4 c) {
        // Reinterpret whole vectors: this compiler folds a bit_cast of a single
        // ext-vector element (v[i], v.y, ...) to element 0.
        const f32x4 af = __builtin_bit_cast(f32x4, a), bf = __builtin_bit_cast(f32x4, b);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(af[0], bf[0], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(af[1], bf[1], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(af[2], bf[2], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(af[3], bf[3], c, 0, 0, 0);
        return c;
    }
};

// LDS tiles: rows of 128 bytes (8 chunks of 16 bytes); chunk kc of row r sits
// at slot kc ^ (r & 7) so that the 16-byte fragment reads of 8 consecutive rows
// hit 8 different bank groups.
__device__ __forceinline__ int lds_off(int row, int kc) { return row * 128 + ((kc ^ (row & 7)) << 4); }

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

}  // namespace lyc
