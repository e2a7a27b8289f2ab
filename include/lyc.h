/*
 * lyc.h -- C ABI of the MI355X (gfx950) fused LoRA-bypass linear.
 *
 * The library computes, on one GPU,
 *
 *   lyc_lora_linear_fwd:  y = round_out( x.W^T + scale * round_c(x.down^T) . up^T + b )
 *   lyc_linear_fwd:       y = round_out( round_out(x.W^T) + b )
 *
 * with the dtype policy of the LyCORIS "Precision" page (section "Dtype
 * policy"): the compute dtype c is the 16-bit type when any operand is
 * 16-bit, else fp32; the output dtype is the promotion of every operand's
 * dtype; fp16 together with bf16 is refused.  Accumulation is fp32 under
 * every policy.  h = x.down^T is rounded to the compute (storage) dtype
 * before the second dot, as the eager two-Linear chain does (same page,
 * "Measured accuracy"); the bypass is folded into the same fp32
 * accumulators as x.W^T, so the product up.down (Delta W) never exists
 * ("VRAM" section of the same page).  The plain affine form rounds the
 * projection before adding the bias and never fuses the bias across that
 * rounding (Luminal FP16 page, "What Was Fixed").  Rounding is IEEE
 * round-to-nearest-even; subnormals are kept.
 *
 * Conventions shared by every call:
 *  - dtype codes: LYC_F16, LYC_BF16, LYC_F32.  A bias dtype of 0 means "no
 *    bias" and requires bias == NULL.
 *  - Layouts are row-major and contiguous: x [M,K], W [N,K] (the nn.Linear
 *    layout), down [rank,K], up [N,rank], b [N], y [M,N].
 *  - Pointers x, w, down, up, b, y and workspace are DEVICE pointers on the
 *    device that owns `stream`.  The caller owns every buffer; the library
 *    allocates, frees and synchronises nothing.  Inputs are only read.  y and
 *    the workspace must not overlap any input or each other.
 *  - x and W must be 16-byte aligned and K a multiple of 8 (16-byte rows);
 *    down, up, b and y need only element alignment.  The workspace must be
 *    256-byte aligned and at least the size the matching *_workspace_size
 *    call reports.  Its contents on entry do not matter.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls are
 *    asynchronous on that stream and deterministic (fixed reduction order, no
 *    atomics in any result path).
 *  - Every argument is checked before any GPU work is queued: a call that
 *    returns an error has launched nothing and written nothing.  M == 0 or
 *    N == 0 is a valid empty call (nothing launched).  K == 0 gives the
 *    empty-sum result (y = round(b)).
 *  - No call throws, aborts or prints.
 */
#ifndef LYC_H
#define LYC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { LYC_F16 = 1, LYC_BF16 = 2, LYC_F32 = 3 };

enum {
    LYC_OK = 0,
    LYC_ERR_MIXED_HALF = 1,     /* fp16 and bf16 operands in one call (a caller bug) */
    LYC_ERR_INVALID_ARG = 2,    /* null pointer, negative size, unknown dtype code, ... */
    LYC_ERR_DTYPE_MISMATCH = 3, /* y_dt is not the resolved output dtype */
    LYC_ERR_UNSUPPORTED = 4,    /* K not a multiple of 8, misaligned x/W, rank > 256, sizes too large */
    LYC_ERR_HIP = 5,            /* the HIP runtime refused a launch */
    LYC_ERR_WORKSPACE = 6,      /* workspace missing, too small or not 256-byte aligned */
    LYC_ERR_IO = 7,             /* tuning table file could not be read, parsed or written */
    LYC_ERR_SCRATCH = 8         /* the problem needs more scratch than lyc_lora_linear_fwd_noalloc holds */
};

/*
 * Resolve the dtype policy over the dtypes of the operands present in a call
 * (x, W, b if any, down and up for the LoRA form) -- LyCORIS "Precision"
 * page, "Dtype policy".
 *   operand_dtypes: host array of n dtype codes (n >= 1).
 *   compute, output: host out-parameters (may be NULL), written on success.
 * Returns LYC_OK, LYC_ERR_MIXED_HALF (fp16 with bf16; nothing written) or
 * LYC_ERR_INVALID_ARG (n < 1, NULL array, unknown code).  Host only.
 */
int lyc_resolve_dtypes(const int* operand_dtypes, int n, int* compute, int* output);

/*
 * Workspace bytes lyc_linear_fwd needs for this problem: for 16-bit compute
 * the projection guard's counts and, where at least 256 output tiles of
 * 64 x 64 keep every CU busy, the hi/lo split of W_c (per 64-k block) and its
 * row norms from a preparation pass (with fewer tiles the contraction splits
 * W itself, in one launch), plus compute-dtype copies of fp32 operands that
 * feed a 16-bit contraction.  Returns the same argument errors as
 * lyc_linear_fwd.
 */
int lyc_linear_workspace_size(int64_t M, int64_t N, int64_t K, int x_dt, int w_dt, int bias_dt,
                              size_t* bytes);

/*
 * Plain affine forward with a declared rounding boundary (Luminal FP16
 * page, "What Was Fixed"): p = x_c.W_c^T (fp32 MFMA steps summed in fp64),
 * p rounded to the output dtype exactly as its exact value rounds (a guard
 * re-evaluates in fp64 every element near a rounding midpoint), then
 * y = round_out(p + b).  bias may be NULL (bias_dt 0): y = round_out(p).
 */
int lyc_linear_fwd(const void* x, int x_dt, const void* w, int w_dt, const void* bias, int bias_dt,
                   void* y, int y_dt, int64_t M, int64_t N, int64_t K,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * The plain affine form with W prepared once: weights kept as prepared data
 * next to their stored values ("Mixed-Precision Kernels" explainer, "The
 * Three-Tier Storage Pattern").  lyc_linear_prepare writes into the caller's
 * workspace (lyc_linear_workspace_size bytes for the same M, N, K and
 * dtypes, 256-byte aligned) what lyc_linear_fwd derives from W on every
 * call: W's compute-dtype copy when W is fp32 under 16-bit compute, and,
 * where the contraction takes W split beforehand, W_c's hi/lo split and row
 * norms.  lyc_linear_fwd_prepared is lyc_linear_fwd without those launches
 * (one launch where x needs no cast): it reads them from the workspace and W
 * itself only to re-evaluate guarded elements.  The caller keeps W and that
 * workspace unchanged between the two calls (lyc_linear_fwd with the same W,
 * shapes and dtypes also leaves the workspace prepared); a workspace
 * prepared for another W gives wrong results, which the library cannot
 * detect.  y is bitwise the result of lyc_linear_fwd.  Calls that share a
 * workspace are ordered by their stream.  Arguments and errors as
 * lyc_linear_fwd (lyc_linear_prepare reads no x, bias or y).
 */
int lyc_linear_prepare(const void* w, int w_dt, int x_dt, int bias_dt, int64_t M, int64_t N, int64_t K,
                       void* workspace, size_t workspace_bytes, void* stream);
int lyc_linear_fwd_prepared(const void* x, int x_dt, const void* w, int w_dt, const void* bias, int bias_dt,
                            void* y, int y_dt, int64_t M, int64_t N, int64_t K,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * Workspace bytes lyc_lora_linear_fwd needs.  It holds the rounded h
 * [M, r_pad] in the compute dtype (r_pad: the rank rounded up to 16 -- under
 * 16-bit compute only --, 32, 64, 128 or 256), compute-dtype copies of down and up (rank padded with zeros), for
 * 16-bit compute the hi/lo split of down_c and its row norms used by the h
 * guard, a counter, and compute-dtype copies of fp32 x/W when they feed a
 * 16-bit contraction.  Returns the same argument errors as
 * lyc_lora_linear_fwd.
 */
int lyc_lora_linear_workspace_size(int64_t M, int64_t N, int64_t K, int64_t rank, int x_dt, int w_dt,
                                   int bias_dt, int down_dt, int up_dt, size_t* bytes);

/*
 * LoRA-bypass forward (LyCORIS "Precision" page, "Dtype policy", "Measured
 * accuracy" and "VRAM"):
 *   h   = x_c . down_c^T           exact to within the rounding decision:
 *                                  h is rounded once, to nearest even, from
 *                                  its exact value (a guard re-evaluates in
 *                                  fp64 every element whose fp32-partial sum
 *                                  lies near a rounding midpoint)
 *   h_r = round_c(h)
 *   y   = round_out( x_c.W_c^T + scale * h_r.up_c^T + b )   fp32 accumulation,
 *                                                           one final rounding
 * where _c denotes an operand rounded (to nearest even) to the compute dtype.
 * scale is a host value applied as an fp32 multiply of the bypass sum.
 * rank == 0 is allowed (no bypass; down/up may be NULL).
 */
int lyc_lora_linear_fwd(const void* x, int x_dt, const void* w, int w_dt, const void* bias, int bias_dt,
                        const void* down, int down_dt, const void* up, int up_dt, int64_t rank, double scale,
                        void* y, int y_dt, int64_t M, int64_t N, int64_t K,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * The same forward with W's compute-dtype copy kept by the caller
 * ("Mixed-Precision Kernels" explainer, "The Three-Tier Storage Pattern": the
 * fp32 master weights and their 16-bit working copy are both carried; with W
 * frozen, as in LoRA training, the copy is made once instead of per call).
 *   w_c:  [N][K], W rounded to nearest even to the compute dtype (for an fp32 W
 *         under a 16-bit policy; otherwise W itself), 16-byte aligned; it must
 *         not overlap y (LYC_ERR_INVALID_ARG).
 *   w_dt: W's own (master) dtype: it enters the dtype policy as in
 *         lyc_lora_linear_fwd, so y's dtype is unchanged.
 * The workspace size comes from lyc_lora_linear_wc_workspace_size (no W copy);
 * lyc_lora_workspace_layout gives the same offsets for both forwards.  Given
 * w_c = round_c(W), results are identical to lyc_lora_linear_fwd's.
 */
int lyc_lora_linear_wc_workspace_size(int64_t M, int64_t N, int64_t K, int64_t rank, int x_dt, int w_dt,
                                      int bias_dt, int down_dt, int up_dt, size_t* bytes);
int lyc_lora_linear_fwd_wc(const void* x, int x_dt, const void* w_c, int w_dt, const void* bias, int bias_dt,
                           const void* down, int down_dt, const void* up, int up_dt, int64_t rank, double scale,
                           void* y, int y_dt, int64_t M, int64_t N, int64_t K, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * The LoRA-bypass forward for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, checks, kernels and results as
 * lyc_lora_linear_fwd, without the workspace: the scratch the kernels need
 * (the size lyc_lora_linear_workspace_size reports) lives in a static device
 * array of LYC_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it
 * runs on, from the first call on that GPU until the process ends.
 *   - Allocates nothing: no hipMalloc, hipFree or allocating library routine.
 *     The caller still passes x, w, down, up, bias and y.  The first call on a
 *     GPU looks up the array's device address (hipGetSymbolAddress, with that
 *     GPU current, the caller's current device restored after).
 *   - Problems whose scratch need exceeds LYC_NOALLOC_SCRATCH_BYTES are
 *     refused with LYC_ERR_SCRATCH before any GPU work.
 *   - Every call on a GPU shares that GPU's array and leaves its contents
 *     behind; each call clears what must start at zero (the guard counter)
 *     with a kernel of its own.  Calls that overlap on one GPU (other streams,
 *     other host threads) race on the array: serialise them.
 *   - stream: the array of the stream's device is used (NULL: the current
 *     device's).
 * Returns the codes of lyc_lora_linear_fwd, LYC_ERR_SCRATCH, or LYC_ERR_HIP
 * when the array's address cannot be looked up.
 */
#define LYC_NOALLOC_SCRATCH_BYTES (64u << 20)
int lyc_lora_linear_fwd_noalloc(const void* x, int x_dt, const void* w, int w_dt, const void* bias, int bias_dt,
                                const void* down, int down_dt, const void* up, int up_dt, int64_t rank, double scale,
                                void* y, int y_dt, int64_t M, int64_t N, int64_t K, void* stream);

/*
 * Where lyc_lora_linear_fwd leaves its intermediate results inside the
 * workspace, for inspection after the call has completed on its stream:
 *   h_offset:  byte offset of h_r, [M][h_ld] in the compute dtype (columns
 *              >= rank are zero);
 *   h_ld:      leading dimension of h_r in elements (r_pad);
 *   flagged_offset: byte offset of `*flagged_slots` uint32 counts whose sum
 *              is the number of h elements that the rounding guard
 *              re-evaluated during the last call: in fp64 after the split
 *              contraction (one count; one per workgroup at rank 16 with down
 *              in the 16-bit compute dtype, which the contraction then splits
 *              itself), or, for few token rows (M <= 128 and
 *              M * r_pad * K <= 2^25, h as one fp64 dot per element), by a
 *              compensated re-summation (one count per workgroup); every
 *              slot is written by each call;
 *   flagged_slots: their number.
 * Any out-pointer may be NULL.  Same argument errors as the size query.
 */
int lyc_lora_workspace_layout(int64_t M, int64_t N, int64_t K, int64_t rank, int x_dt, int w_dt, int bias_dt,
                              int down_dt, int up_dt, size_t* h_offset, int64_t* h_ld, size_t* flagged_offset,
                              int64_t* flagged_slots);

/*
 * Where lyc_linear_fwd keeps its guard counts inside the workspace:
 *   flagged_offset: byte offset of `*flagged_slots` uint32 counts (one per
 *              workgroup of the contraction, each written by it) whose
 *              sum is the number of
 *              projection elements the rounding guard re-evaluated in fp64
 *              during the last call (16-bit compute; all 0 when the output is
 *              fp32, which needs no guard);
 *   flagged_slots: their number (0 under fp32 compute: nothing is written).
 * Any out-pointer may be NULL.  Same argument errors as the size query.
 */
int lyc_linear_workspace_layout(int64_t M, int64_t N, int64_t K, int x_dt, int w_dt, int bias_dt,
                                size_t* flagged_offset, int64_t* flagged_slots);

/*
 * LoRA merge (LyCORIS "Precision" page: "Dtype policy", whose "input" is here
 * the original weight, and the merge figure of "Measured accuracy"):
 *   W' = round_out( W + scale * up_c . down_c )
 * with W [N,K] (the nn.Linear layout), down [rank,K], up [N,rank], all
 * row-major and contiguous, W' [N,K].  The compute dtype c and the output
 * dtype are resolved over (W, down, up) by the dtype policy; up and down are
 * rounded to c, W keeps its stored value (it is not a matmul operand, like
 * the bias of the forward).  The rank-sum runs in fp32 (exact products of
 * 16-bit factors), scale * sum + W is one fp32 fused multiply-add, and that
 * is rounded once to the output dtype (round to nearest even).
 * rank == 0 gives W' = round_out(W) (down/up may be NULL).
 *  - out_dt must equal the resolved output dtype (LYC_ERR_DTYPE_MISMATCH).
 *  - out may be w itself (in-place merge; then out_dt == w_dt, else
 *    LYC_ERR_INVALID_ARG); any other overlap of out with w is
 *    LYC_ERR_INVALID_ARG.  out must not overlap down, up or the workspace.
 *  - Pointers need element alignment only; 16-byte-aligned rows with K a
 *    multiple of 4 take the vector path.  N, K <= 2^30 and N*K <= 2^38,
 *    rank <= 256, else LYC_ERR_UNSUPPORTED.  N == 0 or K == 0 launches
 *    nothing.  scale must be finite and within the fp32 range.
 *  - The workspace (256-byte aligned, lyc_lora_merge_workspace_size bytes,
 *    0 when rank == 0) receives compute-dtype copies of down^T and up.  When
 *    down and up are already in a 16-bit compute dtype, rank and K are
 *    multiples of 8 and both are 16-byte aligned, they are read as stored
 *    and the workspace is left untouched (it is still required).
 * The same stream, ownership and error conventions as the forward calls.
 */
int lyc_lora_merge_workspace_size(int64_t N, int64_t K, int64_t rank, int w_dt, int down_dt, int up_dt,
                                  size_t* bytes);
int lyc_lora_merge_fwd(const void* w, int w_dt, const void* down, int down_dt, const void* up, int up_dt,
                       int64_t rank, double scale, void* out, int out_dt, int64_t N, int64_t K,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * LoRA-bypass backward (LyCORIS "Precision" page: "Dtype policy" -- each
 * gradient comes back in its own leaf's dtype -- and "VRAM" -- h is
 * recomputed, up.down and its gradient are never formed).  Given dy [M,N],
 * the gradient of y, with c the compute dtype of the dtype policy over
 * (x, W, b, down, up, dy):
 *   h_r   = round_c( x_c . down_c^T )                 recomputed as the forward computes it
 *   gh_r  = round_c( scale * dy_c . up_c )            [M, rank], rounded once from its exact
 *                                                     value (the same guard as h)
 *   dx    = round_x( dy_c . W_c + gh_r . down_c )     [M, K] in x's dtype
 *   dDown = round_down( gh_r^T . x_c )                [rank, K] in down's dtype
 *   dUp   = round_up( scale * dy_c^T . h_r )          [N, rank] in up's dtype
 * fp32 accumulation, one final rounding each (dUp: the fp32 sum times scale
 * in fp32, then rounded).  W and the bias are the frozen base layer: no
 * gradient; bias_dt (0: none) only enters the policy, so that c is the
 * forward's.  Layouts as in the forward; dy row-major [M,N].
 *  - dx, d_down, d_up: device outputs; a NULL one is not computed (and what
 *    only it needs is skipped).  They must not overlap any input or each
 *    other (LYC_ERR_INVALID_ARG).  Element alignment suffices.
 *  - K and N multiples of 8; M, N, K <= 2^20, rank <= 256
 *    (LYC_ERR_UNSUPPORTED).  x (when it is read in the compute dtype, i.e.
 *    x_dt == c) and dy (likewise) must be 16-byte aligned; W, down, up need
 *    element alignment.  M == 0 gives zero dDown and dUp.
 *  - The workspace (256-byte aligned) holds h_r, gh_r, the guard's splits and
 *    norms, compute-dtype copies of fp32 x/dy, and transposed compute-dtype
 *    copies of W and down (for dx).  Under 16-bit compute the token
 *    contractions (dDown, dUp) read x, dy, h_r and gh_r as stored, the token
 *    index as their contraction rows (each of them below 1 GiB); under fp32
 *    compute (or larger operands) transposed copies of those are made in the
 *    workspace too.  Its size comes from
 *    lyc_lora_linear_bwd_workspace_size with `want` = 1 (dx) | 2 (dDown) |
 *    4 (dUp), the set of non-NULL outputs of the call (| 8 for
 *    lyc_lora_linear_bwd_wt, which needs no W^T copy; | 16 for
 *    lyc_lora_linear_bwd_saved given h_r, which needs no h region).
 * Same stream, ownership and error conventions as the forward.
 */
int lyc_lora_linear_bwd_workspace_size(int64_t M, int64_t N, int64_t K, int64_t rank, int x_dt, int w_dt,
                                       int bias_dt, int down_dt, int up_dt, int dy_dt, int want, size_t* bytes);
int lyc_lora_linear_bwd(const void* x, int x_dt, const void* w, int w_dt, int bias_dt, const void* down,
                        int down_dt, const void* up, int up_dt, int64_t rank, double scale, const void* dy,
                        int dy_dt, void* dx, void* d_down, void* d_up, int64_t M, int64_t N, int64_t K,
                        void* workspace, size_t workspace_bytes, void* stream);
/*
 * The same backward with a caller-kept transposed weight, for LoRA training
 * where W is frozen across steps (LyCORIS "Precision" page, "VRAM": the
 * frozen base weight is used as stored, nothing of its size is rebuilt per
 * step).  w_t is W_c^T: [K][N] row-major in the compute dtype c of the call,
 * each element W[n][k] rounded to nearest even to c (the caller rounds and
 * transposes once; for 16-bit W already in c it is the plain transpose).  It
 * must be 16-byte aligned and must not overlap any output.  w_dt is still the
 * stored dtype of W (a policy operand).  dx reads w_t in place: the
 * workspace skips the W^T copy -- its size comes from
 * lyc_lora_linear_bwd_workspace_size with bit 8 added to `want`.  Results
 * are identical to lyc_lora_linear_bwd's.
 */
int lyc_lora_linear_bwd_wt(const void* x, int x_dt, const void* w_t, int w_dt, int bias_dt, const void* down,
                           int down_dt, const void* up, int up_dt, int64_t rank, double scale, const void* dy,
                           int dy_dt, void* dx, void* d_down, void* d_up, int64_t M, int64_t N, int64_t K,
                           void* workspace, size_t workspace_bytes, void* stream);
/*
 * The backward with what a training step keeps from its forward: the
 * forward's h_r = round_c(x_c . down_c^T), which dUp = round_up(scale * dy_c^T
 * . h_r) reads (the forward computes it anyway; LyCORIS "Precision" page,
 * "Measured accuracy": h is rounded to the storage dtype before its second
 * dot, so the saved value is the one the backward needs), and optionally the
 * caller-kept W_c^T of lyc_lora_linear_bwd_wt.
 *   w, w_t: at most one non-NULL (LYC_ERR_INVALID_ARG otherwise); w_t as for
 *           lyc_lora_linear_bwd_wt.  Neither is read unless dx is wanted.
 *   h_r:    NULL (recomputed, as lyc_lora_linear_bwd does), or [M][r_pad] in
 *           the compute dtype, 16-byte aligned, exactly as lyc_lora_linear_fwd
 *           left it in its workspace (h_offset and h_ld = r_pad from
 *           lyc_lora_workspace_layout) for the same x, down and dtypes: no h
 *           pass runs.  Read only when dUp is wanted; it must not overlap an
 *           output (LYC_ERR_INVALID_ARG).
 * The workspace size comes from lyc_lora_linear_bwd_workspace_size with bit
 * 16 added to `want` when h_r is given (and 8 when w_t is).  Given the
 * forward's h_r, results are identical to lyc_lora_linear_bwd's.
 */
int lyc_lora_linear_bwd_saved(const void* x, int x_dt, const void* w, const void* w_t, int w_dt, int bias_dt,
                              const void* down, int down_dt, const void* up, int up_dt, const void* h_r,
                              int64_t rank, double scale, const void* dy, int dy_dt, void* dx, void* d_down,
                              void* d_up, int64_t M, int64_t N, int64_t K, void* workspace, size_t workspace_bytes,
                              void* stream);
/*
 * Where lyc_lora_linear_bwd leaves h_r and gh_r in its workspace (both
 * [M][ld] in the compute dtype; SIZE_MAX when the call set `want` does not
 * compute them) and the uint32 count of gh elements its guard re-evaluated
 * in fp64 (16-bit compute; else SIZE_MAX).  Same argument errors as the size query.
 */
int lyc_lora_linear_bwd_workspace_layout(int64_t M, int64_t N, int64_t K, int64_t rank, int x_dt, int w_dt,
                                         int bias_dt, int down_dt, int up_dt, int dy_dt, int want,
                                         size_t* h_offset, size_t* gh_offset, int64_t* ld, size_t* flagged_offset);

/*
 * DoRA (the LyCORIS "Precision" page, "VRAM": the DoRA row norms are the small
 * state the kernels cache, one fp32 value per row).  The merged weight
 * V = W + scale * up_c . down_c (the merge's definition and dtype policy over
 * (W, down, up), never stored) and its row norms
 *   norm_n = || V[n, :] ||_2 ,
 * then the DoRA forward, with the magnitude vector m [N]:
 *   y = round_out( (m_n / norm_n) * (x_c.W_c^T + scale * round_c(x_c.down_c^T).up_c^T)_n + b_n )
 * -- the LoRA forward with each output feature's sum scaled before the bias
 * is added.  The dtype policy runs over (x, W, b, down, up, m).
 * lyc_dora_norms: norms [N] fp32 (device), computed tile by tile from W and
 *   the factors (fp32 sums of squares per tile, added in tile order, square
 *   root); the workspace (256-byte aligned, lyc_dora_norms_workspace_size
 *   bytes) holds the factors' compute-dtype copies and the per-tile sums.
 *   norms must not overlap W.  Argument errors as lyc_lora_merge_fwd.
 * lyc_dora_linear_fwd: the arguments of lyc_lora_linear_fwd plus magnitude
 *   (m_dt, element-aligned) and norms (fp32, as lyc_dora_norms writes them);
 *   the gain m_n / norm_n is one fp32 division, applied to the fp32 sum.
 *   Workspace: lyc_dora_linear_workspace_size (the LoRA forward's plus the
 *   gain vector).  Errors as lyc_lora_linear_fwd.
 */
int lyc_dora_norms_workspace_size(int64_t N, int64_t K, int64_t rank, int w_dt, int down_dt, int up_dt,
                                  size_t* bytes);
int lyc_dora_norms(const void* w, int w_dt, const void* down, int down_dt, const void* up, int up_dt, int64_t rank,
                   double scale, float* norms, int64_t N, int64_t K, void* workspace, size_t workspace_bytes,
                   void* stream);
int lyc_dora_linear_workspace_size(int64_t M, int64_t N, int64_t K, int64_t rank, int x_dt, int w_dt, int bias_dt,
                                   int down_dt, int up_dt, int m_dt, size_t* bytes);
int lyc_dora_linear_fwd(const void* x, int x_dt, const void* w, int w_dt, const void* bias, int bias_dt,
                        const void* down, int down_dt, const void* up, int up_dt, const void* magnitude, int m_dt,
                        const float* norms, int64_t rank, double scale, void* y, int y_dt, int64_t M, int64_t N,
                        int64_t K, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Tile planner and measured pick for the LoRA forward's main contraction
 * (LyCORIS "Backend Selection" page, "Tile selection": an analytic model
 * shortlists candidates, the shortlist is timed once, best of three, and the
 * winner is kept in memory and in a table file keyed by device, op, bucketed
 * shape and dtype).
 *
 * lyc_gemm_plan: the shortlist for an M x N x K product with a fold of rf
 *   (padded rank) steps in compute dtype compute_dt, best first -- first the
 *   pick the forward makes on its own, then the other (tile, K split) pairs
 *   in the order of the model's time, which counts rounds of workgroups over
 *   the device's CUs at its MFMA rate, a per-tile re-read penalty, and the
 *   partial sums' round trip through HBM at its rate for a K split (the
 *   rates lyc_device_rates reports).  Writes up to max_out (at most 7)
 *   entries into the host arrays tile_n, tile_m (output tile: rows of W x rows
 *   of x), ksplit, cost_us (any may be NULL) and their number into *count.
 *   Host only.
 * lyc_device_rates: the planner's model of the current device: its CU
 *   count (hipDeviceAttributeMultiprocessorCount) and its dense MFMA rates
 *   with 16-bit and fp32 operands (flop/s) and HBM rate (bytes/s).  Until
 *   measured on the device (*measured = 0) the rates are MI355X's published
 *   peaks per CU (2.5 PFLOP/s and 157.3 TFLOP/s over 256 CUs) times the CU
 *   count, and 8 TB/s; without a device, 256 CUs.  Any pointer may be NULL.
 * lyc_measure_device_rates: measures those rates on the device of `stream`
 *   and keeps them for the planner (per device, for the process): a 256 MiB
 *   device-to-device copy (read + write bytes over time) and MFMA loops of
 *   16 waves per CU (v_mfma_f32_16x16x32_f16, whose published peak bf16
 *   shares, and v_mfma_f32_16x16x4_f32), each the best of three timed runs.  BLOCKS the host; allocates 512 MiB of
 *   device memory for the copy and frees it.  LYC_ERR_HIP on a HIP failure.
 * lyc_lora_linear_tune: the same arguments as lyc_lora_linear_fwd (whose
 *   output y it overwrites), plus the winner's tile, split and time (any
 *   may be NULL) and, in cand_ms (NULL or 7 doubles), the best time of
 *   each shortlisted candidate in lyc_gemm_plan's order.  It first measures
 *   the device's rates (lyc_measure_device_rates) if not yet done, so the
 *   shortlist is ordered by them.  Runs the whole
 *   forward once and then three times timed
 *   with each shortlisted configuration on `stream`, and stores the fastest
 *   under the key of this device and shape; later lyc_lora_linear_fwd calls
 *   with that key use it.  BLOCKS the host until the timed runs end (the one
 *   call of the library that synchronises).  With the environment variable
 *   LYC_KERNEL_TUNE=off (or 0) it times nothing and stores the planner's
 *   first candidate.  The workspace is the forward's (its size covers every
 *   shortlisted K split).
 * lyc_tuning_key: the key of a forward call on the current device into buf
 *   (e.g. "gfx950-256cu|lora_fwd|M4096|N3072|K3072|r16|c1|o1": device, op, M
 *   rounded up to a power of two (at least 16), N, K, padded rank, compute
 *   and output dtypes).  LYC_ERR_HIP without a current device,
 *   LYC_ERR_INVALID_ARG if buf is NULL or shorter than the key + 1.
 * lyc_tuning_lookup: *found = 1 and the stored pick if the table holds one
 *   for that call on the current device, else *found = 0.
 * lyc_tuning_save / lyc_tuning_load: the table as JSON, one entry per line
 *   ({"key": ..., "tile_n": ..., "tile_m": ..., "ksplit": ..., "ms": ...}).
 *   Loading merges into the table (*entries = the number read) and takes
 *   nothing from a file with a malformed entry (LYC_ERR_IO).  A stored pick
 *   the forward cannot run (a tile without an instance for the compute dtype,
 *   a split beyond its workspace) is ignored by the forward.
 * lyc_tuning_clear / lyc_tuning_count: empty the table / its size.
 * The table is process-wide and guarded by a mutex.
 */
int lyc_gemm_plan(int64_t M, int64_t N, int64_t K, int64_t rf, int compute_dt, int max_out, int* count, int* tile_n,
                  int* tile_m, int* ksplit, double* cost_us);
int lyc_device_rates(int64_t* cus, double* mfma16_flops, double* mfma32_flops, double* hbm_bytes_per_s,
                     int* measured);
int lyc_measure_device_rates(void* stream);
int lyc_lora_linear_tune(const void* x, int x_dt, const void* w, int w_dt, const void* bias, int bias_dt,
                         const void* down, int down_dt, const void* up, int up_dt, int64_t rank, double scale,
                         void* y, int y_dt, int64_t M, int64_t N, int64_t K, void* workspace, size_t workspace_bytes,
                         void* stream, int* tile_n, int* tile_m, int* ksplit, double* best_ms, double* cand_ms);
int lyc_tuning_key(int64_t M, int64_t N, int64_t K, int64_t rank, int x_dt, int w_dt, int bias_dt, int down_dt,
                   int up_dt, char* buf, size_t len);
int lyc_tuning_lookup(int64_t M, int64_t N, int64_t K, int64_t rank, int x_dt, int w_dt, int bias_dt, int down_dt,
                      int up_dt, int* found, int* tile_n, int* tile_m, int* ksplit);
int lyc_tuning_save(const char* path);
int lyc_tuning_load(const char* path, int* entries);
int lyc_tuning_clear(void);
int lyc_tuning_count(void);

/*
 * Output tile (rows of W x rows of x) that the forward calls use for an
 * M x N problem in compute dtype compute_dt; one workgroup computes one tile.
 * Host only.  Returns LYC_ERR_INVALID_ARG for negative sizes or an unknown
 * dtype code.
 */
int lyc_gemm_tile(int64_t M, int64_t N, int compute_dt, int* tile_n, int* tile_m);

/*
 * Per-kernel device time, recorded with HIP events around each kernel the
 * forward calls launch (the measurement discipline of the Luminal FP16 page,
 * "One Identical Implementation Through Timing and Profiling": per-kernel
 * durations of the very launches being timed).  Off unless started.
 *   lyc_profile_begin(capacity): create `capacity` event pairs (host call;
 *     no device memory) and record every following launch, up to capacity.
 *     Returns LYC_ERR_INVALID_ARG for capacity < 1, LYC_ERR_HIP if the events
 *     cannot be created.
 *   lyc_profile_end(total_ms, launches): wait for the recorded events, write
 *     per kernel kind k (LYC_KERNEL_CAST .. LYC_KERNEL_GEMM) the summed
 *     duration in ms and the launch count into the host arrays
 *     total_ms[LYC_KERNEL_KINDS], launches[LYC_KERNEL_KINDS] (either may be
 *     NULL), free the events, stop recording.
 * Process-wide state: begin/end must not race with each other.
 */
enum {
    LYC_KERNEL_CAST = 0,   /* fp32 operand -> 16-bit compute copy */
    LYC_KERNEL_PREP = 1,   /* low-rank factor / W preparation (copies, split, norms; the merge's down^T/up copies) */
    LYC_KERNEL_HPASS = 2,  /* h = x.down^T, its rounding guard and fp64 re-evaluations */
    LYC_KERNEL_GEMM = 3,   /* the main contraction and epilogue (plain affine: the exactly rounded projection;
                              merge: the merge kernel) */
    LYC_KERNEL_KINDS = 4
};
int lyc_profile_begin(int capacity);
int lyc_profile_end(double* total_ms, int* launches);

/* Static, NUL-terminated description of a status code. */
const char* lyc_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* LYC_H */
