// merge.hip -- the LoRA merge W' = round_out(W + scale * up_c . down_c)
// (LyCORIS "Precision" page: "Dtype policy" with the original weight as the
// input operand, and the merge figure of "Measured accuracy"), and the DoRA
// row norms of the merged weight (same page, "VRAM").
//
// The merge streams W in and W' out once: 4-6 bytes per element against
// 2 r flops, so it is bound by HBM for every rank the library takes.  Two
// forms:
//  * streaming (merge_stream_kernel, below): 16-bit W, W' and factors read
//    as stored, rank up to 128 -- one workgroup per CU walks 16-row tiles
//    down a band of 512 columns, W staged through LDS several tiles ahead,
//    down's band held as MFMA fragments in registers;
//  * general (merge_kernel): any dtypes, ranks and alignments.  One
//    workgroup owns a 128 x 128 tile of W:
//   1. the first rank chunk of up_c and down^T_c is requested, then the whole
//      W tile, 16 bytes per lane in row order (coalesced), into registers,
//      non-temporally (W and W' pass through once; the rank operands, re-read
//      by every tile, stay in L2);
//   2. while W is in flight, the rank contraction runs on MFMA from LDS
//      (chunks of 128 bytes of every operand row, 16-byte slots swizzled;
//      or, with down and up read as stored, down's rank rows as a
//      contraction-major tile read through the transposing LDS read);
//   3. the fp32 accumulators go through LDS once more, so that
//   4. each lane meets the W elements it loaded: W' = fma(scale, acc, W),
//      rounded once, stored 16 bytes per lane in row order.
//   67.5 KiB of LDS and at most 256 VGPRs: two workgroups per CU.
#include "lyc_device.h"
#include "merge.h"

namespace lyc {

namespace {
constexpr int MT = 128;                 // W rows (n) per workgroup
constexpr int MC = 128;                 // W columns (k) per workgroup
constexpr int XS = MC + 4;              // exchange row stride in floats (conflict-free 16-byte writes)
constexpr int LDS = MT / 2 * XS * 4;    // 33792 bytes; the operand chunk needs (MT + MC) * 128 = 32768
constexpr int BOFF = MC * 128;          // byte offset of the up_c chunk behind the down^T_c chunk
static_assert((MT + MC) * 128 <= LDS, "operand chunk fits the exchange buffer");
}  // namespace

// One rank chunk (128 bytes of every row) of the 128 down^T_c rows (ra) and
// the 128 up_c rows (rb) of a tile: 8 rows per 32-thread group, one 16-byte
// slot per thread.
//
// RAW (down and up as the caller stores them, already in the compute dtype):
// chunk c of the A side is rank rows 64c .. 64c+63 of down [rank][K] over the
// tile's 128 k columns, kept as a contraction-major tile (256-byte rows,
// 16-byte chunks permuted by tswz) for the transposing LDS read; rows past the
// rank and columns past K are sent out of range explicitly (no offset is
// formed for them, so none can wrap back into down) and read 0.  The B side
// reads up [N][rank] rows with their own stride rowb_u (rank elements).
template <bool RAW>
__device__ __forceinline__ void merge_chunk_loads(i32x4 (&st)[8], __amdgpu_buffer_rsrc_t ra,
                                                  __amdgpu_buffer_rsrc_t rb, int c, uint32_t rowb, int orow,
                                                  int okc, int tid, int64_t K, int64_t k0, uint32_t rowb_u,
                                                  int64_t rank) {
    const uint32_t byte = (uint32_t)c * 128 + okc * 16;
    if constexpr (RAW) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int i = q * 256 + tid, r = i >> 4, s = i & 15;
            const int64_t k = k0 + 8 * (s ^ tswz<16>(r));
            const int64_t rr = 64 * c + r;
            st[q] = buf_load16(ra, (rr < rank && k < K) ? (uint32_t)((rr * K + k) * 2) : OOB);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
            st[4 + q] = buf_load16(rb, byte < rowb_u ? (uint32_t)(q * 32 + orow) * rowb_u + byte : OOB);
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) st[q] = buf_load16(ra, byte < rowb ? (uint32_t)(q * 32 + orow) * rowb + byte : OOB);
#pragma unroll
        for (int q = 0; q < 4; ++q)
            st[4 + q] = buf_load16(rb, byte < rowb ? (uint32_t)(q * 32 + orow) * rowb + byte : OOB);
    }
}

// Chunk c to LDS (16-byte slots swizzled per row), then its one or two
// 64-byte MFMA substeps: this wave's 64 k x 64 n quadrant.
template <class CT, bool RAW>
__device__ __forceinline__ void merge_chunk_mma(char* smem, const i32x4 (&st)[8], f32x4 (&acc)[4][4], int c,
                                                uint32_t rowb, int orow, int okc, int lane, int wn, int wk, int tid) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        if (RAW && q < 4) {
            const int i = q * 256 + tid;
            *(i32x4*)(smem + (i >> 4) * 256 + (i & 15) * 16) = st[q];
        } else {
            *(i32x4*)(smem + (q < 4 ? 0 : BOFF) + lds_off((q & 3) * 32 + orow, okc)) = st[q];
        }
    }
    lds_barrier();
    const int nsub = (uint32_t)c * 128 + 64 < rowb ? 2 : 1;
    for (int s = 0; s < nsub; ++s) {
        i32x4 fa[4], fb[4];
        const int kc = 4 * s + (lane >> 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (RAW) fa[i] = frag_t<MC>(smem, 32 * s, 64 * wk + 16 * i, lane);
            else fa[i] = *(const i32x4*)(smem + lds_off(64 * wk + 16 * i + (lane & 15), kc));
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) fb[j] = *(const i32x4*)(smem + BOFF + lds_off(64 * wn + 16 * j + (lane & 15), kc));
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = CT::step(fa[i], fb[j], acc[i][j]);
    }
}

// The A-side resource of a tile: prepared, its 128 rows of down^T_c; RAW, all
// of down [rank][K] (the offsets carry the tile's columns)
template <bool RAW>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t merge_rsrc_a(const MergeParams& p, int64_t k0, int64_t ka,
                                                               uint32_t rowb) {
    if constexpr (RAW) return make_rsrc_uniform(p.down_raw, (uint32_t)(p.rank * p.K * 2));
    else return make_rsrc_uniform((const char*)p.dt_c + k0 * rowb, (uint32_t)ka * rowb);
}

// NORM: instead of storing W', each tile adds up v^2 over its columns for
// every row and writes that partial sum to norm_partial[tile column][n] (the
// DoRA row norms of the merged weight, which is never stored).
template <class CT, bool WF, bool OF, bool VEC, bool NORM, bool RAW>
__global__ __launch_bounds__(256, (WF || !VEC) ? 2 : 3) void merge_kernel(MergeParams p, int tiles_k) {
    __shared__ __attribute__((aligned(16))) char smem[LDS];
    // a thread's share of the tile: E consecutive elements of one row per pass
    constexpr int E = (WF || OF) ? 4 : 8;
    constexpr int CPR = MC / E, RPP = 256 / CPR, P = MT / RPP;
    constexpr int WES = WF ? 4 : 2;
    constexpr int WW = E * WES / 4;     // 32-bit words of W per pass
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wn = wave >> 1, wk = wave & 1;

    // workgroups are dealt round-robin over the 8 XCDs: give each XCD a
    // contiguous row-major range of tiles (they share up_c rows in its L2)
    const int nblk = gridDim.x, per = nblk >> 3, rem = nblk & 7;
    const int xcd = blockIdx.x & 7, loc = blockIdx.x >> 3;
    const int l = xcd * per + (xcd < rem ? xcd : rem) + loc;
    const int64_t n0 = (int64_t)(l / tiles_k) * MT, k0 = (int64_t)(l % tiles_k) * MC;

    // 1a. the first rank chunk of the operands (range-checked buffer loads:
    //     rows past N or K and bytes past the padded rank read 0)
    const uint32_t rowb = (uint32_t)p.r_pad * CT::es;
    const int nchunk = (int)((rowb + 127) / 128);
    const int64_t ka = p.K - k0 < MC ? p.K - k0 : MC, nb_ = p.N - n0 < MT ? p.N - n0 : MT;
    const uint32_t rowb_u = RAW ? (uint32_t)p.rank * CT::es : rowb;   // up's row stride
    const auto ra = merge_rsrc_a<RAW>(p, k0, ka, rowb);
    const auto rb = make_rsrc_uniform((const char*)(RAW ? p.up_raw : p.uc) + n0 * rowb_u, (uint32_t)nb_ * rowb_u);
    const int orow = tid >> 3, okc = tid & 7;   // operand row (of 32 per load) and 16-byte slot
    // (unconditional: without a rank every offset is out of range and reads 0;
    // a branch here would cost the exact wait counts below)
    i32x4 st[8];
    merge_chunk_loads<RAW>(st, ra, rb, 0, rowb, orow, okc, tid, p.K, k0, rowb_u, p.rank);

    // 1b. the W tile, behind the operand chunk in the memory queue.  VEC: K
    //     is a multiple of E and the rows are aligned, so a lane's chunk is
    //     either wholly inside W or wholly outside (then it reads a valid
    //     chunk and stores nothing).  Otherwise, element loads at clamped
    //     indices.  (No branch between the two: a join here would make the
    //     compiler's wait before the first LDS write cover the W loads too.)
    const int prow = tid / CPR, pcol = (tid % CPR) * E;
    uint32_t wv[P][WW];
#pragma unroll
    for (int q = 0; q < P; ++q) {
        const int64_t n = n0 + q * RPP + prow;
        if constexpr (VEC) {
            const int64_t k = k0 + pcol;
            const char* src = (const char*)p.w + ((n < p.N && k < p.K) ? n * p.K + k : 0) * WES;
            if constexpr (WW == 4) {
                const i32x4 t = __builtin_nontemporal_load((const i32x4*)src);
#pragma unroll
                for (int e = 0; e < 4; ++e) wv[q][e] = (uint32_t)t[e];
            } else {
                const i32x2 t = __builtin_nontemporal_load((const i32x2*)src);
                wv[q][0] = (uint32_t)t[0];
                wv[q][1] = (uint32_t)t[1];
            }
        } else {
            uint32_t raw[E];
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const int64_t k = k0 + pcol + e;
                const int64_t idx = (n < p.N && k < p.K) ? n * p.K + k : 0;
                raw[e] = WF ? ((const uint32_t*)p.w)[idx] : (uint32_t)((const uint16_t*)p.w)[idx];
            }
#pragma unroll
            for (int t = 0; t < WW; ++t) wv[q][t] = WF ? raw[t] : (raw[2 * t] | (raw[2 * t + 1] << 16));
        }
    }

    // 2. rank contraction: acc[i][j] holds, per 16 x 16 block, k rows of
    //    down^T_c (A side) by n columns of up_c (B side).  Chunk 0 is peeled
    //    off the loop so that its wait covers its own loads only, not the W
    //    loads issued after them.
    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    merge_chunk_mma<CT, RAW>(smem, st, acc, 0, rowb, orow, okc, lane, wn, wk, tid);
    for (int c = 1; c < nchunk; ++c) {
        merge_chunk_loads<RAW>(st, ra, rb, c, rowb, orow, okc, tid, p.K, k0, rowb_u, p.rank);
        lds_barrier();   // every wave is done reading the previous chunk
        merge_chunk_mma<CT, RAW>(smem, st, acc, c, rowb, orow, okc, lane, wn, wk, tid);
    }

    // 3-4. in two halves of 64 rows: the accumulators of the waves that own
    //      the half go to LDS as X[n][k] (lane: 4 consecutive k of one n), then
    //      every lane finishes the elements of that half it loaded:
    //      W' = round_out(fma(scale, acc, W))
    float* X = (float*)smem;
    constexpr int OES = OF ? 4 : 2;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
    lds_barrier();
    if (wn == half) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            *(f32x4*)(X + (16 * j + (lane & 15)) * XS + 64 * wk + 16 * i + 4 * (lane >> 4)) = acc[i][j];
    }
    lds_barrier();
#pragma unroll
    for (int qq = 0; qq < P / 2; ++qq) {
        const int q = half * (P / 2) + qq;
        const int rl = q * RPP + prow;
        const int rx = qq * RPP + prow;
        float a[E];
#pragma unroll
        for (int h = 0; h < E / 4; ++h) {
            const f32x4 t = *(const f32x4*)(X + rx * XS + pcol + 4 * h);
#pragma unroll
            for (int e = 0; e < 4; ++e) a[4 * h + e] = t[e];
        }
        float v[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
            float w;
            if constexpr (WF) {
                w = __builtin_bit_cast(float, wv[q][e]);
            } else {
                const uint16_t b = (uint16_t)(wv[q][e >> 1] >> ((e & 1) * 16));
                w = CT::dt == DT_F16 ? f16_to_f32(b) : bf16_to_f32(b);
            }
            v[e] = __builtin_fmaf(p.scale, a[e], w);
        }
        const int64_t n = n0 + rl;
        if constexpr (NORM) {
            // squares of this lane's in-range elements, then the sum over the
            // CPR lanes of the row (a fixed butterfly: deterministic)
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const bool in = n < p.N && k0 + pcol + e < p.K;
                ss = __builtin_fmaf(in ? v[e] : 0.f, in ? v[e] : 0.f, ss);
            }
#pragma unroll
            for (int o = CPR / 2; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 64);
            if (tid % CPR == 0 && n < p.N) p.norm_partial[(int64_t)(l % tiles_k) * p.N + n] = ss;
            continue;
        }
        uint32_t o[E * OES / 4];
        if constexpr (OF) {
#pragma unroll
            for (int e = 0; e < E; ++e) o[e] = __builtin_bit_cast(uint32_t, v[e]);
        } else {
#pragma unroll
            for (int t = 0; t < E / 2; ++t)
                o[t] = CT::dt == DT_F16 ? pack_f16x2(v[2 * t], v[2 * t + 1]) : pack_bf16x2(v[2 * t], v[2 * t + 1]);
        }
        if constexpr (VEC) {
            if (n < p.N && k0 + pcol < p.K)
                __builtin_nontemporal_store(i32x4{(int)o[0], (int)o[1], (int)o[2], (int)o[3]}, (i32x4*)((char*)p.out + (n * p.K + k0 + pcol) * OES));
        } else if (n < p.N) {
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const int64_t k = k0 + pcol + e;
                if (k >= p.K) continue;
                if constexpr (OF) ((uint32_t*)p.out)[n * p.K + k] = o[e];
                else ((uint16_t*)p.out)[n * p.K + k] = (uint16_t)(o[e >> 1] >> ((e & 1) * 16));
            }
        }
    }
    }
}

// ---- streaming form: 16-bit W, W' and factors, read as stored ----------------
// One workgroup of 8 waves per CU owns a band of 512 columns of W and walks a
// run of 16-row tiles down it, so that W is read and written in pieces of 1
// KiB per row.  down's 512 columns of the band are turned into MFMA fragments
// once (staged in LDS, read by the transposing LDS read) and stay in
// registers; each tile of W (16 rows x 1 KiB) and the tile's 16 rows of up
// are staged in LDS by direct-to-LDS loads NS-1 tiles ahead.  Wave w owns the
// tile's columns 64w .. 64w+63: after its MFMAs every lane holds 4
// consecutive k of one row per 16 x 16 block, an 8-byte piece of the staged W
// row, so W' = round_out(fma(scale, acc, W)) is written back over it in
// place, and the tile then leaves LDS one row per wave store.  The norm mode
// sums v^2 per row and tile instead (one partial per row and band, added up
// after the next tile's barrier).
namespace {
constexpr int ST_N = 16, ST_K = 512;         // tile rows (n) and band columns (k)
constexpr int ST_RB = ST_K * 2;              // bytes of a staged W row
constexpr int ST_W = ST_N * ST_RB;           // bytes of a staged W tile
constexpr int ST_STORES = ST_W / 16 / 512;   // 16-byte stores per thread and tile
// up rows of a tile: one sub-tile of 16 rows x 128 bytes per 64 of the padded rank
template <int RP> constexpr int st_sub() { return RP <= 64 ? 1 : RP / 64; }
template <int RP> constexpr int st_bytes() { return ST_W + st_sub<RP>() * ST_N * 128; }
template <int RP> constexpr int st_ql() { return st_bytes<RP>() / 1024; }   // 1 KiB loads per tile
// stages: at most 4 (3 tiles in flight per CU, about 60 KiB).  Filling the
// LDS (6 or 7 tiles in flight) was slower, and so were two workgroups per CU
// with 3 stages each: with more requests outstanding the HBM stream loses
// locality (bf16 8192 x 8192 r128: merge 49.8 -> 47.6 us, row norms 36.5 ->
// 33.5 us against 7 stages; 59.4 and 35.7 us with two workgroups; a plain
// read sweep likewise runs fastest with one 16-byte load per lane in flight)
template <int RP> constexpr int st_ns() { return (159 * 1024) / st_bytes<RP>() > 4 ? 4 : (159 * 1024) / st_bytes<RP>(); }
template <int RP> constexpr int st_stages() { return st_ns<RP>() * st_bytes<RP>(); }
// down's band: max(RP, 32) rank rows of 1 KiB, behind the stages where that
// fits, else over them (it is read once, before the stages fill)
template <int RP> constexpr int st_setup() { return (RP < 32 ? 32 : RP) * ST_RB; }
template <int RP> constexpr bool st_apart() { return st_stages<RP>() + st_setup<RP>() + 1024 <= 150 * 1024; }
template <int RP> constexpr int st_setup_at() { return st_apart<RP>() ? st_stages<RP>() : 0; }
template <int RP> constexpr int st_red_at() {
    return st_apart<RP>() ? st_stages<RP>() + st_setup<RP>()
                          : (st_stages<RP>() > st_setup<RP>() ? st_stages<RP>() : st_setup<RP>());
}
template <int RP> constexpr int st_lds() { return st_red_at<RP>() + 2 * 8 * ST_N * 4; }
}  // namespace

// s_waitcnt vmcnt(min(n, N)) for a wave-uniform n (a smaller count only waits longer)
template <int N>
__device__ __forceinline__ void wait_vm_dyn(int n) {
    if constexpr (N == 0) {
        wait_vm<0>();
    } else {
        if (n >= N) wait_vm<N>();
        else wait_vm_dyn<N - 1>(n);
    }
}

// Direct-to-LDS loads of one tile: W's 16 rows over the band, one row per
// load (chunk c of row r in slot c ^ (r & 15) of its 1 KiB row), and up's 16
// rows, 64 rank values per sub-tile (chunk c of row r in slot c ^ (r & 7),
// lds_off), two loads per sub-tile.  Wave w takes loads w, w + 8, ...
// Offsets past K, the rank or the tile's rows read zeros.
// rw and ru cover all of W and up; wb and ub are the byte offsets of the
// tile's first row in them (rows past N then lie past the resource: zeros).
template <int RP>
__device__ __forceinline__ void stream_issue(char* stage, __amdgpu_buffer_rsrc_t rw, __amdgpu_buffer_rsrc_t ru,
                                             uint32_t wb, uint32_t ub, int64_t kb0, int64_t K, int64_t rank, int wave,
                                             int lane) {
    constexpr int QL = st_ql<RP>();
#pragma unroll
    for (int u = 0; u < (QL + 7) / 8; ++u) {
        const int q = wave + 8 * u;   // loads 0..15: W; then up, 2 per sub-tile
        if (q >= QL) break;
        auto* dst = (__attribute__((address_space(3))) void*)(stage + q * 1024);
        if (u < ST_N / 8) {
            const int row = q, c = lane ^ (row & 15);
            const int64_t k = kb0 + 8 * c;
            const uint32_t off = k < K ? (uint32_t)(((int64_t)row * K + k) * 2) : OOB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, dst, 16, off == OOB ? OOB : off + wb, 0, 0, 0);
        } else {
            const int qu = q - ST_N, sub = qu >> 1, row = (qu & 1) * 8 + (lane >> 3);
            const int64_t r = 64 * sub + 8 * ((lane & 7) ^ (row & 7));
            const uint32_t off = r < rank ? (uint32_t)(((int64_t)row * rank + r) * 2) : OOB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ru, dst, 16, off == OOB ? OOB : off + ub, 0, 0, 0);
        }
    }
}

template <class CT, int RP, bool NORM>
__global__ __launch_bounds__(512, 1) void merge_stream_kernel(MergeParams p, int runs) {
    constexpr int SB = st_bytes<RP>(), NS = st_ns<RP>();
    constexpr int RS = RP < 32 ? 1 : RP / 32;   // 32-wide rank steps
    constexpr int QW = st_ql<RP>() / 8;         // loads per wave and tile, at least
    __shared__ __attribute__((aligned(16))) char sm[st_lds<RP>()];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // the wave's 64 columns of the band

    // the workgroup's band of columns and run of row tiles
    const int band = (int)blockIdx.x / runs, run = (int)blockIdx.x % runs;
    const int64_t kb0 = (int64_t)band * ST_K;
    const int NT = (int)((p.N + ST_N - 1) / ST_N);
    const int t0 = (int)((int64_t)NT * run / runs), nt = (int)((int64_t)NT * (run + 1) / runs) - t0;

    // down's band (rank rows past its end and columns past K read 0), then its
    // fragments for the wave's 64 columns into registers
    i32x4 af[4][RS];
    {
        constexpr int DR = RP < 32 ? 32 : RP;
        char* setup = sm + st_setup_at<RP>();
        const auto rd = make_rsrc_uniform(p.down_raw, (uint32_t)(p.rank * p.K * 2));
#pragma unroll
        for (int u = 0; u < DR / 8; ++u) {
            const int row = wave + 8 * u;
            const int64_t k = kb0 + 8 * (lane ^ tswz<64>(row));
            const uint32_t off = (row < p.rank && k < p.K) ? (uint32_t)(((int64_t)row * p.K + k) * 2) : OOB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, (__attribute__((address_space(3))) void*)(setup + row * 1024),
                                                     16, off, 0, 0, 0);
        }
        wait_vm<0>();
        lds_barrier();
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int rs = 0; rs < RS; ++rs) af[kb][rs] = frag_t<ST_K>(setup, 32 * rs, 64 * wave + 16 * kb, lane);
        // the stages may overlay the band: every wave has its fragments first
        lds_barrier();
    }

    // whole-matrix resources, made once (W, up and W' below 2 GiB); a tile's
    // rows are a byte offset in them
    const auto rw = make_rsrc_uniform(p.w, (uint32_t)(p.N * p.K * 2));
    const auto ru = make_rsrc_uniform(p.up_raw, (uint32_t)(p.N * p.rank * 2));
    const uint32_t wrow = (uint32_t)(ST_N * p.K * 2), urow = (uint32_t)(ST_N * p.rank * 2);   // bytes per tile
    for (int i = 0; i < NS - 1; ++i)
        if (i < nt) stream_issue<RP>(sm + i * SB, rw, ru, (uint32_t)(t0 + i) * wrow, (uint32_t)(t0 + i) * urow, kb0,
                                     p.K, p.rank, wave, lane);
    // norm mode: per-row sums of the 8 waves, [tile parity][wave][16 rows]; a
    // tile's are added up after the next tile's barrier
    float* red = (float*)(sm + st_red_at<RP>());

    // unrolled by the stage count: every stage address is a constant offset
    for (int i0 = 0; i0 < nt; i0 += NS)
#pragma unroll
    for (int u = 0; u < NS; ++u) {
        const int i = i0 + u;
        if (i >= nt) break;
        // tile i has landed once at most the operations issued after its loads
        // are outstanding: the loads of the tiles after it and, storing, the
        // stores of the tiles before it issued since
        const int la = nt - 1 - i < NS - 2 ? nt - 1 - i : NS - 2;
        const int sa = NORM ? 0 : (i < NS - 1 ? i : NS - 1);
        wait_vm_dyn<QW * (NS - 2) + (NORM ? 0 : ST_STORES * (NS - 1))>(QW * la + ST_STORES * sa);
        lds_barrier();   // every wave's loads of tile i are in; tile i-1's stage is free
        if (NORM && i > 0 && tid < ST_N) {
            const float* rp = red + ((i - 1) & 1) * (8 * ST_N);
            const int64_t n = (int64_t)(t0 + i - 1) * ST_N + tid;
            float t = rp[tid];
#pragma unroll
            for (int w = 1; w < 8; ++w) t += rp[w * ST_N + tid];
            if (n < p.N) p.norm_partial[(int64_t)band * p.N + n] = t;
        }
        if (i + NS - 1 < nt)
            stream_issue<RP>(sm + ((u + NS - 1) % NS) * SB, rw, ru, (uint32_t)(t0 + i + NS - 1) * wrow,
                             (uint32_t)(t0 + i + NS - 1) * urow, kb0, p.K, p.rank, wave, lane);
        char* st = sm + u * SB;
        const int64_t n0 = (int64_t)(t0 + i) * ST_N;

        i32x4 bq[RS];
        const int row = lane & 15;
#pragma unroll
        for (int rs = 0; rs < RS; ++rs)
            bq[rs] = *(const i32x4*)(st + ST_W + (rs >> 1) * (ST_N * 128) + lds_off(row, (rs & 1) * 4 + (lane >> 4)));
        // the lane's 4 pieces of the staged W row, all read before any is
        // written back (a store first would make the compiler wait for it
        // before the next read), then the 4 column blocks' MFMAs interleaved
        char* wa[4];
        i32x2 wv[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const int cb = 128 * wave + 32 * kb + 8 * (lane >> 4);   // byte of the lane's 4 columns in the row
            wa[kb] = st + row * ST_RB + (((cb >> 4) ^ row) << 4) + (cb & 15);
            wv[kb] = *(const i32x2*)wa[kb];
        }
        f32x4 acc[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) acc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int rs = 0; rs < RS; ++rs)
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) acc[kb] = CT::step(af[kb][rs], bq[rs], acc[kb]);
        float ss = 0.f;   // norm mode: the lane's sum of v^2 over its 16 columns of the tile
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint16_t b = (uint16_t)((uint32_t)wv[kb][e >> 1] >> ((e & 1) * 16));
                const float w = CT::dt == DT_F16 ? f16_to_f32(b) : bf16_to_f32(b);
                v[e] = __builtin_fmaf(p.scale, acc[kb][e], w);
            }
            if constexpr (NORM) {
                // (rows past N and columns past K are 0: W, up and down all
                // read zeros there)
#pragma unroll
                for (int e = 0; e < 4; ++e) ss = __builtin_fmaf(v[e], v[e], ss);
            } else {
                const uint32_t o0 = CT::dt == DT_F16 ? pack_f16x2(v[0], v[1]) : pack_bf16x2(v[0], v[1]);
                const uint32_t o1 = CT::dt == DT_F16 ? pack_f16x2(v[2], v[3]) : pack_bf16x2(v[2], v[3]);
                *(i32x2*)wa[kb] = i32x2{(int)o0, (int)o1};
            }
        }
        if constexpr (NORM) {
            // the 4 lanes of each row (a fixed butterfly); the waves' sums are
            // added in order after the next barrier
            // (gfx950 row swaps: the same sums as shuffles with lanes l^16 and
            // l^32, which went through the LDS crossbar; the pair of results is
            // reinterpreted whole, as a bit_cast of one element of a vector
            // folds to element 0)
            const uint32_t u = __builtin_bit_cast(uint32_t, ss);
            const f32x2_t a = __builtin_bit_cast(f32x2_t, __builtin_amdgcn_permlane16_swap(u, u, false, false));
            ss = a[0] + a[1];
            const uint32_t w = __builtin_bit_cast(uint32_t, ss);
            const f32x2_t b = __builtin_bit_cast(f32x2_t, __builtin_amdgcn_permlane32_swap(w, w, false, false));
            ss = b[0] + b[1];
            if (lane < 16) red[(i & 1) * (8 * ST_N) + wave * ST_N + row] = ss;
        } else {
            lds_barrier();   // the tile's merged values are all in LDS
            // out one 1 KiB row per wave store, nontemporal (W' is not read
            // again here; 46.8 against 52.0 us at bf16 8192 x 8192); every store
            // is issued (past K or past the tile's rows its offset is out of
            // range), so the wait counts above hold
            const auto ro = make_rsrc_uniform((const char*)p.out, (uint32_t)(p.N * p.K * 2));
#pragma unroll
            for (int h = 0; h < ST_STORES; ++h) {
                const int r = 8 * h + wave, c = lane;
                const i32x4 v = *(const i32x4*)(st + r * ST_RB + ((c ^ r) << 4));
                const int64_t k = kb0 + 8 * c;
                const uint32_t off = k < p.K ? (uint32_t)(((int64_t)r * p.K + k) * 2) + (uint32_t)(t0 + i) * wrow : OOB;
                __builtin_amdgcn_raw_buffer_store_b128(v, ro, off, 0, 2);   // nontemporal
            }
        }
    }
    if constexpr (NORM) {
        lds_barrier();
        if (nt > 0 && tid < ST_N) {
            const float* rp = red + ((nt - 1) & 1) * (8 * ST_N);
            const int64_t n = (int64_t)(t0 + nt - 1) * ST_N + tid;
            float t = rp[tid];
#pragma unroll
            for (int w = 1; w < 8; ++w) t += rp[w * ST_N + tid];
            if (n < p.N) p.norm_partial[(int64_t)band * p.N + n] = t;
        }
    }
}

bool merge_streams(int c_dt, const MergeParams& p) {
    if (c_dt != DT_F16 && c_dt != DT_BF16) return false;
    if (p.w_dt != c_dt || (p.norm_partial == nullptr && p.out_dt != c_dt)) return false;
    return p.vec && p.down_raw != nullptr && p.up_raw != nullptr && p.rank > 0 && p.r_pad <= 128 &&
           (p.N + ST_N) * p.K * 2 < ((int64_t)1 << 31) && p.rank * p.K * 2 < ((int64_t)1 << 31) &&
           (p.N + ST_N) * p.rank * 2 < ((int64_t)1 << 31);
}

// runs (of row tiles) per band of 512 columns: about one workgroup per CU in all
static int merge_stream_runs(const MergeParams& p) {
    const int64_t bands = (p.K + ST_K - 1) / ST_K, nt = (p.N + ST_N - 1) / ST_N;
    int64_t runs = 256 / bands;
    if (runs > nt) runs = nt;
    return runs < 1 ? 1 : (int)runs;
}

template <class CT, int RP>
static hipError_t run_merge_stream(const MergeParams& p, hipStream_t s) {
    const int runs = merge_stream_runs(p);
    const dim3 g((unsigned)(((p.K + ST_K - 1) / ST_K) * runs));
    if (p.norm_partial != nullptr) hipLaunchKernelGGL((merge_stream_kernel<CT, RP, true>), g, dim3(512), 0, s, p, runs);
    else hipLaunchKernelGGL((merge_stream_kernel<CT, RP, false>), g, dim3(512), 0, s, p, runs);
    return hipGetLastError();
}

template <class CT>
static hipError_t run_merge_stream_rp(const MergeParams& p, hipStream_t s) {
    switch (p.r_pad) {
    case 16: return run_merge_stream<CT, 16>(p, s);
    case 32: return run_merge_stream<CT, 32>(p, s);
    case 64: return run_merge_stream<CT, 64>(p, s);
    case 128: return run_merge_stream<CT, 128>(p, s);
    default: return hipErrorInvalidValue;
    }
}

// DoRA row norms: the tiles' partial sums of squares of each row, added in
// tile order, then the square root (fp32)
__global__ __launch_bounds__(256) void norm_finish_kernel(const float* partial, int tiles_k, int64_t N, float* norms) {
    const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (n >= N) return;
    // 16 loads in flight at a time, the adds still in tile order
    float s = 0.f;
    for (int t0 = 0; t0 < tiles_k; t0 += 16) {
        float v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = partial[(int64_t)(t0 + i < tiles_k ? t0 + i : 0) * N + n];
#pragma unroll
        for (int i = 0; i < 16; ++i) s += t0 + i < tiles_k ? v[i] : 0.f;
    }
    norms[n] = (float)__builtin_sqrt((double)s);
}

hipError_t launch_norm_finish(int c_dt, const MergeParams& p, hipStream_t s) {
    if (p.N <= 0) return hipSuccess;
    // partials per row: one per band of 256 columns (streaming form), else per 128-column tile
    const int tiles_k = (int)((p.K + (merge_streams(c_dt, p) ? ST_K : MC) - 1) / (merge_streams(c_dt, p) ? ST_K : MC));
    hipLaunchKernelGGL(norm_finish_kernel, dim3((unsigned)((p.N + 255) / 256)), dim3(256), 0, s, p.norm_partial,
                       tiles_k, p.N, p.norms);
    return hipGetLastError();
}

// DoRA gain g_n = m_n / norm_n (fp32)
__global__ __launch_bounds__(256) void dora_gain_kernel(const void* m, int m_dt, const float* norms, int64_t N,
                                                        float* gain) {
    const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (n < N) gain[n] = load_as_f32(m, m_dt, n) / norms[n];
}

hipError_t launch_dora_gain(const void* m, int m_dt, const float* norms, int64_t N, float* gain, hipStream_t s) {
    if (N <= 0) return hipSuccess;
    hipLaunchKernelGGL(dora_gain_kernel, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, s, m, m_dt, norms, N, gain);
    return hipGetLastError();
}

// down [rank][K] -> down^T_c [K][r_pad] (rounded to the compute dtype, zero
// columns from rank on), 32 columns of down per workgroup through LDS so that
// both the reads and the writes run along rows; the remaining workgroups copy
// up [N][rank] -> up_c [N][r_pad], one element per thread.
template <class T>
__device__ __forceinline__ float widen(T v, int dt) {
    if constexpr (sizeof(T) == 4) return __builtin_bit_cast(float, v);
    else return dt == DT_F16 ? f16_to_f32(v) : bf16_to_f32(v);
}
__device__ __forceinline__ void put_c(void* dst, int64_t i, float v, int c_dt) {
    if (c_dt == DT_F32) ((float*)dst)[i] = v;
    else ((uint16_t*)dst)[i] = c_dt == DT_F16 ? f32_to_f16(v) : f32_to_bf16(v);
}

template <class TD, class TU>
__global__ __launch_bounds__(256) void merge_prep_kernel(MergePrepParams p, int down_blocks) {
    __shared__ float T[32][257];
    const int tid = threadIdx.x;
    if ((int)blockIdx.x < down_blocks) {
        const int64_t k0 = (int64_t)blockIdx.x * 32;
        const int kk = tid & 31, jg = tid >> 5;
        const int64_t k = k0 + kk;
        const TD* d = (const TD*)p.down;
        const int64_t kc = k < p.K ? k : p.K - 1;   // clamped: every load is issued unmasked
#pragma unroll 8
        for (int j = jg; j < p.rank; j += 8) {
            const float v = widen(d[(int64_t)j * p.K + kc], p.down_dt);
            T[kk][j] = k < p.K ? v : 0.f;
        }
        __syncthreads();
        const int sh = __builtin_ctz((unsigned)p.r_pad);
        for (int i = tid; i < 32 * p.r_pad; i += 256) {
            const int r = i >> sh, j = i & (p.r_pad - 1);
            if (k0 + r < p.K) put_c(p.dt_c, (k0 + r) * p.r_pad + j, j < p.rank ? T[r][j] : 0.f, p.c_dt);
        }
        return;
    }
    const int sh = __builtin_ctz((unsigned)p.r_pad);
    const int64_t total = p.N * (int64_t)p.r_pad;
    const int64_t stride = (int64_t)(gridDim.x - down_blocks) * 256;
    const TU* u = (const TU*)p.up;
    for (int64_t i = (int64_t)(blockIdx.x - down_blocks) * 256 + tid; i < total; i += stride) {
        const int64_t n = i >> sh;
        const int j = (int)(i & (p.r_pad - 1));
        const float v = widen(u[n * p.rank + (j < p.rank ? j : 0)], p.up_dt);
        put_c(p.uc, i, j < p.rank ? v : 0.f, p.c_dt);
    }
}

hipError_t launch_merge_prep(const MergePrepParams& p, hipStream_t s) {
    const int down_blocks = (int)((p.K + 31) / 32);
    int64_t up_blocks = (p.N * (int64_t)p.r_pad + 255) / 256;
    if (up_blocks > 8192) up_blocks = 8192;
    if (up_blocks < 1) up_blocks = 1;
    const dim3 g((unsigned)(down_blocks + up_blocks));
    const bool d32 = p.down_dt == DT_F32, u32 = p.up_dt == DT_F32;
    if (d32 && u32) hipLaunchKernelGGL((merge_prep_kernel<uint32_t, uint32_t>), g, dim3(256), 0, s, p, down_blocks);
    else if (d32) hipLaunchKernelGGL((merge_prep_kernel<uint32_t, uint16_t>), g, dim3(256), 0, s, p, down_blocks);
    else if (u32) hipLaunchKernelGGL((merge_prep_kernel<uint16_t, uint32_t>), g, dim3(256), 0, s, p, down_blocks);
    else hipLaunchKernelGGL((merge_prep_kernel<uint16_t, uint16_t>), g, dim3(256), 0, s, p, down_blocks);
    return hipGetLastError();
}

template <class CT, bool WF, bool OF, bool RAW>
static hipError_t run_merge_raw(const MergeParams& p, hipStream_t s) {
    const int tiles_n = (int)((p.N + MT - 1) / MT), tiles_k = (int)((p.K + MC - 1) / MC);
    const dim3 g((unsigned)(tiles_n * tiles_k));
    if (p.norm_partial != nullptr) {
        if (p.vec) hipLaunchKernelGGL((merge_kernel<CT, WF, OF, true, true, RAW>), g, dim3(256), 0, s, p, tiles_k);
        else hipLaunchKernelGGL((merge_kernel<CT, WF, OF, false, true, RAW>), g, dim3(256), 0, s, p, tiles_k);
        return hipGetLastError();
    }
    if (p.vec) hipLaunchKernelGGL((merge_kernel<CT, WF, OF, true, false, RAW>), g, dim3(256), 0, s, p, tiles_k);
    else hipLaunchKernelGGL((merge_kernel<CT, WF, OF, false, false, RAW>), g, dim3(256), 0, s, p, tiles_k);
    return hipGetLastError();
}

// RAW (down and up read as stored) for 16-bit compute only
template <class CT, bool WF, bool OF>
static hipError_t run_merge(const MergeParams& p, hipStream_t s) {
    if constexpr (CT::dt != DT_F32) {
        if (p.down_raw != nullptr) return run_merge_raw<CT, WF, OF, true>(p, s);
    } else {
        if (p.down_raw != nullptr) return hipErrorInvalidValue;
    }
    return run_merge_raw<CT, WF, OF, false>(p, s);
}

hipError_t launch_merge(int c_dt, const MergeParams& p, hipStream_t s) {
    if (merge_streams(c_dt, p))
        return c_dt == DT_F16 ? run_merge_stream_rp<CF16>(p, s) : run_merge_stream_rp<CBF16>(p, s);
    const bool wf = p.w_dt == DT_F32, of = p.out_dt == DT_F32;
    if (wf && !of) return hipErrorInvalidValue;   // the policy promotes an fp32 W to an fp32 W'
    switch (c_dt) {
    case DT_F16: return wf ? run_merge<CF16, true, true>(p, s) : of ? run_merge<CF16, false, true>(p, s)
                                                                   : run_merge<CF16, false, false>(p, s);
    case DT_BF16: return wf ? run_merge<CBF16, true, true>(p, s) : of ? run_merge<CBF16, false, true>(p, s)
                                                                     : run_merge<CBF16, false, false>(p, s);
    case DT_F32: return (wf && of) ? run_merge<CF32, true, true>(p, s) : hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
    }
}

}  // namespace lyc
